// Intra-chunk stage: everything about a chunk that does not depend on the
// state entering it.  One 512-thread workgroup (8 waves) per (chunk, head);
// all chunks of all heads run in parallel.
//
// For a chunk of n <= C tokens (rows r), with G the inclusive cumulative
// log2-gate inside the chunk and gamma_r = 2^{G_r}:
//   a1  G = cumsum(g * log2(e))                        (wave prefix scan)
//   a2  A_ij = beta_i 2^{G_i - G_j} (k_i . k_j), j < i   (k1, on MFMA)
//       Aqk_ij = scale 2^{G_i - G_j} (q_i . k_j), j <= i
//   a3  Ainv = (I + A)^{-1}                              (k2)
//       16x16 diagonal blocks by forward substitution, then
//       X_IJ = -X_II sum_{m=J}^{I-1} A_Im X_mJ, block row by block row
//   a4  W = Ainv diag(beta) diag(gamma) K,  U = Ainv diag(beta) V   (k3)
// and, for the state pass, Qs = scale diag(gamma) Q and Ks = diag(gamma_C/gamma) K.
// Sources: "TileLang 实战：KDA 从零到一--Gated DeltaNet" §2.2.4 (UT transform,
// eqs. 6-7), §2.2.6 (gated substitutions), §2.3 (eqs. 11-12), §4.1 (log-domain
// cumulative gate, masked before exponentiation), §4.2 (blocked inverse);
// "阅读笔记：DeltaNet 在 FLA 中的代码实现笔记", forward Steps 1-3 (16x16 blocks
// solved by forward substitution and combined block-wise).
//
// Per-key gate (Kimi Delta Attention, "DeltaNet 系列线性注意力变体的推导之旅",
// chunkwise section): every 2^{G_i - G_j} sits inside the sum over the key
// channel d.  Off-diagonal 16x16 blocks (I > J) factor through the first token
// b of block I:  sum_d (k_id 2^{G_id - G_bd}) (k_jd 2^{G_bd - G_jd}), both
// exponents <= 0, so they run on MFMA without overflow.  Inside a diagonal
// block the same holds for its lower-left 8x8 quadrant (rows 8..15, columns
// 0..7) with b its row 8, so that quadrant runs on MFMA too; the two 8x8
// triangles left are summed pair by pair.  gamma and gamma_C/gamma become
// per-channel.
//
// Layout choices: K, Q and V stay row-major (key- or value-contiguous) in
// LDS.  Products that contract over tokens read them with transposing LDS
// loads, and compute X^T rather than X, so that every lane holds 4
// consecutive columns of one output row and stores them to HBM directly.
// beta (and gamma) multiply the columns of Ainv instead of the rows of K, V.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

constexpr int INTRA_THREADS = 512;

template <typename T, int K, int V, int C, bool PK>
struct IntraSmem {
    static constexpr int P = 16 / sizeof(T);  // 16-byte row padding
    static constexpr int LDK = K + P;         // row-major [C][K]
    static constexpr int LDV = V + P;         // row-major [C][V]
    static constexpr int LDC = C + P;         // row-major [C][C] in the element type
    static constexpr int LDA = C + 4;         // fp32 [C][C]
    // per-key gate: fp32 [C][K] rows padded by 8 floats, so that the diagonal
    // blocks' reads (8 rows x 8 interleaved channels per wave) hit 64
    // different banks
    static constexpr int LDG = PK ? K + 8 : 1;
    static constexpr int NB = C / 16;
    // per-key scaled operands, two buffers of SCR_ROWS rows: 32 + C - 16
    // rows for an off-diagonal block row, 3 x C / 2 for the diagonal blocks'
    // quadrants (and >= C)
    static constexpr int SCR_ROWS = (32 + C - 16) > 3 * C / 2 ? 32 + C - 16 : 3 * C / 2;
    static constexpr size_t o_K = 0;
    static constexpr size_t o_Q = o_K + sizeof(T) * C * LDK;
    static constexpr size_t o_V = o_Q + sizeof(T) * C * LDK;
    static constexpr size_t o_A = o_V + sizeof(T) * C * LDV;
    static constexpr size_t o_G = o_A + sizeof(float) * C * LDA;
    static constexpr size_t o_B = o_G + sizeof(float) * C * LDG;
    static constexpr size_t o_E = o_B + sizeof(float) * C;     // 2^{G_r}
    static constexpr size_t o_F = o_E + sizeof(float) * C;     // 2^{G_C-1 - G_r}
    static constexpr size_t o_P = o_F + sizeof(float) * C;
    static constexpr size_t o_S = o_P + sizeof(float) * 4 * 16 * 17;
    static constexpr size_t bytes = o_S + (PK ? 2 * sizeof(T) * SCR_ROWS * LDK : 0);   // two buffers
    // Ainv diag(beta gamma) goes where Q was, Ainv diag(beta) where A was
    static_assert(C * LDC * sizeof(T) <= C * LDK * sizeof(T), "A1 fits the Q region");
    static_assert(C * LDC * sizeof(T) <= C * LDA * sizeof(float), "A2 fits the A region");
};

template <typename T, int K, int V, int C, bool PK, bool STORE_AINV, bool BWD = false>
__global__ __launch_bounds__(INTRA_THREADS) void intra_kernel(IntraLaunch a) {
    typedef IntraSmem<T, K, V, C, PK> L;
    typedef Mma<T> M;
    constexpr int NT = INTRA_THREADS, NW = NT / 64;
    constexpr int LDK = L::LDK, LDV = L::LDV, LDC = L::LDC, LDA = L::LDA, NB = L::NB, LDG = L::LDG;
    constexpr int EV = 16 / sizeof(T);
    constexpr int KS = M::KSTEP;
    __shared__ __attribute__((aligned(16))) char smem[L::bytes];
    T* sK = reinterpret_cast<T*>(smem + L::o_K);
    T* sQ = reinterpret_cast<T*>(smem + L::o_Q);
    T* sV = reinterpret_cast<T*>(smem + L::o_V);
    float* sA = reinterpret_cast<float*>(smem + L::o_A);
    float* sG = reinterpret_cast<float*>(smem + L::o_G);
    float* sB = reinterpret_cast<float*>(smem + L::o_B);
    float* sE = reinterpret_cast<float*>(smem + L::o_E);
    float* sF = reinterpret_cast<float*>(smem + L::o_F);
    float* sP = reinterpret_cast<float*>(smem + L::o_P);
    T* sA1 = sQ;                              // Ainv diag(beta gamma)   (after Q is used)
    T* sA2 = reinterpret_cast<T*>(sA);        // Ainv diag(beta)         (after A is used)

    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    // Workgroups run roughly in id order; ids go to the chunks in decreasing
    // position inside their sequence (all heads of a chunk together), so the
    // first chunks, which the state pass reads first, are written last and
    // are the ones still held in the memory-side cache when it starts.
    const int64_t H = a.H, bid = blockIdx.x, h = bid % H, cr = bid / H;
    // GVA: q and k have Hq heads; value head h reads q/k head h / (H / Hq)
    const int64_t Hq = a.Hq > 0 ? a.Hq : H, hq = h / (H / Hq);
    int64_t c;
    if (a.map.table) {
        c = a.map.max_chunks - 1 - cr;
    } else {
        const int64_t B = a.map.max_chunks / a.map.nt;
        c = (cr % B) * a.map.nt + (a.map.nt - 1 - cr / B);
    }

    // ---- which tokens this chunk covers
    int64_t t0;
    int n;
    if (a.map.table) {
        const int4 e = a.map.table[c];
        t0 = e.x;
        n = e.y;
    } else {
        const int64_t b = c / a.map.nt, j = c - b * a.map.nt;
        t0 = b * a.map.T + j * C;
        n = (int)min((int64_t)C, a.map.T - j * C);
    }
    if (n <= 0) return;
    const int64_t blk = h * a.map.max_chunks + c;   // workspace block index
    const T* q = static_cast<const T*>(a.q);
    const T* k = static_cast<const T*>(a.k);
    const T* v = static_cast<const T*>(a.v);

    // ---- loads: K, Q, V rows, issued before any is used.  Rows past n (tail
    // chunk) repeat row n-1: with beta = 0 there, their rows and columns of
    // A, Ainv diag(beta), W and U come out exactly zero, so they never reach
    // an output, and the loads need no branch.
    constexpr int NKV = C * K / EV, NVV = C * V / EV;
    static_assert(NKV % NT == 0 && NVV % NT == 0, "whole passes");
    constexpr int PKQ = NKV / NT, PV = NVV / NT;
    // the per-key gate first: the gate scan below needs only it, and runs
    // while K, Q and V are still arriving
    constexpr int TPC = NT / K, RPT = C / TPC;   // threads per channel, rows per thread
    float graw[PK ? RPT : 1];
    if constexpr (PK) {
        const int d = tid % K, qq = tid / K;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = qq * RPT + i;
            graw[i] = r < n ? a.g[((t0 + r) * H + h) * K + d] : 0.f;
        }
    }
    u32x4 kr[PKQ], qr[PKQ], vr[PV];
#pragma unroll
    for (int p = 0; p < PKQ; ++p) {
        const int i = tid + NT * p, r = min(i / (K / EV), n - 1), cv = i % (K / EV);
        kr[p] = *reinterpret_cast<const u32x4*>(k + ((t0 + r) * Hq + hq) * K + cv * EV);
        qr[p] = *reinterpret_cast<const u32x4*>(q + ((t0 + r) * Hq + hq) * K + cv * EV);
    }
#pragma unroll
    for (int p = 0; p < PV; ++p) {
        const int i = tid + NT * p, r = min(i / (V / EV), n - 1), cv = i % (V / EV);
        vr[p] = *reinterpret_cast<const u32x4*>(v + ((t0 + r) * H + h) * V + cv * EV);
    }

    // ---- a1: gates and beta; cumulative log2 gate (rows >= n: g = 0, beta = 0)
    if (!PK) {
        if (wave == 0) {
            const int r = lane;
            float gl = 0.f, bt = 0.f;
            if (r < n) {
                const float gr = a.g[(t0 + r) * H + h], br = a.beta[(t0 + r) * H + h];
                gl = ((a.act.flags & ACT_GATE) ? act_log_gate(gr, a.act.A_log[h], a.act.dt_bias[h]) : gr) *
                     LOG2E;
                bt = (a.act.flags & ACT_BETA_SIGMOID) ? act_beta(br, a.act.flags & ACT_BETA_NEG_EIG) : br;
            }
            const float G = wave_incl_scan(gl, lane);
            const float Gc = __shfl(G, C - 1, 64);
            if (r < C) {
                sG[r] = G;
                sB[r] = bt;
                sE[r] = exp2_hw(G);
                sF[r] = exp2_hw(fminf(Gc - G, 0.f));
            }
        }
    } else {
        // per channel d: the inclusive sum over the rows, by all threads.
        // Thread (quarter qq, channel d) loads and scans rows qq*RPT ..
        // (qq+1)*RPT-1 (all its loads in flight together); the quarter totals
        // go through LDS (the sP scratch) and each quarter adds those before it.
        static_assert(TPC * RPT == C && TPC * K <= 4 * 16 * 17, "gate scan split");
        const int d = tid % K, qq = tid / K;
        float gv[RPT];
#pragma unroll
        for (int i = 0; i < RPT; ++i) gv[i] = graw[i];
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = qq * RPT + i;
            float gr = gv[i];
            if (r < n && (a.act.flags & ACT_GATE))
                gr = act_log_gate(gr, a.act.A_log[h], a.act.dt_bias[h * K + d]);
            acc += gr * LOG2E;
            gv[i] = acc;
        }
        sP[qq * K + d] = acc;
        __syncthreads();
        float off = 0.f;
        for (int q2 = 0; q2 < qq; ++q2) off += sP[q2 * K + d];
#pragma unroll
        for (int i = 0; i < RPT; ++i) sG[(qq * RPT + i) * LDG + d] = gv[i] + off;
        for (int r = tid; r < C; r += NT) {
            const float br = r < n ? a.beta[(t0 + r) * H + h] : 0.f;
            sB[r] = r >= n ? 0.f
                    : (a.act.flags & ACT_BETA_SIGMOID) ? act_beta(br, a.act.flags & ACT_BETA_NEG_EIG)
                                                        : br;
        }
    }
    if (a.act.flags & ACT_QK_L2NORM) {   // a row is K / EV consecutive lanes
#pragma unroll
        for (int p = 0; p < PKQ; ++p) {
            kr[p] = l2norm_piece<T, K / EV>(kr[p]);
            qr[p] = l2norm_piece<T, K / EV>(qr[p]);
        }
    }
#pragma unroll
    for (int p = 0; p < PKQ; ++p) {
        const int i = tid + NT * p, r = i / (K / EV), cv = i % (K / EV);
        *reinterpret_cast<u32x4*>(sK + r * LDK + cv * EV) = kr[p];
        *reinterpret_cast<u32x4*>(sQ + r * LDK + cv * EV) = qr[p];
    }
#pragma unroll
    for (int p = 0; p < PV; ++p) {
        const int i = tid + NT * p, r = i / (V / EV), cv = i % (V / EV);
        *reinterpret_cast<u32x4*>(sV + r * LDV + cv * EV) = vr[p];
    }
    __syncthreads();

    // ---- outputs that need only G, Q, K, in MFMA fragment order (one task =
    // one 64-lane x 16-byte group): Qs = scale 2^{G} Q (rows = tokens) and
    // Ks^T = (2^{G_C - G} K)^T (rows = keys), and the cumulative gate.  The
    // backward mode writes Ks (rows = tokens) and Qs^T (rows = keys) as well
    // as Ks^T, and no Qs.
    {
        typedef FragOrder<T> F;
        constexpr int VE = F::VE, KG = F::KG;
        constexpr int NQG = (C / 16) * (K / KG), NKG = (K / 16) * (C / KG);
        T* gqs = static_cast<T*>(a.ws.qs) + blk * C * K;
        T* gks = static_cast<T*>(a.ws.ks) + blk * C * K;
        T* gksr = BWD ? static_cast<T*>(a.ws.ksr) + blk * C * K : nullptr;
        // group `task` of a token-row matrix  f(r) * X[r][d]  (X = sQ or sK)
        auto row_group = [&](const T* sX, bool q_side, T* dst, int task) {
            const int rt = task / (K / KG), sg = task % (K / KG), r = 16 * rt + (lane & 15);
            const T* src = sX + r * LDK + KG * sg;
            float x[VE], f[VE];
            if constexpr (sizeof(T) == 2) {
                const typename M::frag fr = M::load(src, lane);
#pragma unroll
                for (int e = 0; e < VE; ++e) x[e] = (float)fr[e];
            } else {
#pragma unroll
                for (int e = 0; e < VE; ++e) x[e] = Elem<T>::load(src + F::col(lane, e));
            }
#pragma unroll
            for (int e = 0; e < VE; ++e) {
                const int d = KG * sg + F::col(lane, e);
                f[e] = q_side ? a.scale * (PK ? exp2_hw(sG[r * LDG + d]) : sE[r]) * x[e]
                              : (PK ? exp2_hw(fminf(sG[(C - 1) * LDG + d] - sG[r * LDG + d], 0.f))
                                    : sF[r]) * x[e];
            }
            *reinterpret_cast<uint4*>(dst + ((int64_t)task * 64 + lane) * VE) = Vec16<T>::pack(f);
        };
        // group `t` of a key-row matrix  (f(tok) * X[tok][kd])^T
        auto col_group = [&](const T* sX, bool q_side, T* dst, int t) {
            const int rt = t / (C / KG), sg = t % (C / KG);
            const int kd = 16 * rt + (lane & 15);
            float x[VE], f[VE];
            if constexpr (sizeof(T) == 2) {
                const typename M::frag fr = M::load_t(sX + KG * sg * LDK + 16 * rt, LDK, lane);
#pragma unroll
                for (int e = 0; e < VE; ++e) x[e] = (float)fr[e];
            } else {
#pragma unroll
                for (int e = 0; e < VE; ++e)
                    x[e] = Elem<T>::load(sX + (KG * sg + F::col(lane, e)) * LDK + kd);
            }
#pragma unroll
            for (int e = 0; e < VE; ++e) {
                const int tok = KG * sg + F::col(lane, e);
                f[e] = q_side ? a.scale * (PK ? exp2_hw(sG[tok * LDG + kd]) : sE[tok]) * x[e]
                              : (PK ? exp2_hw(fminf(sG[(C - 1) * LDG + kd] - sG[tok * LDG + kd], 0.f))
                                    : sF[tok]) * x[e];
            }
            *reinterpret_cast<uint4*>(dst + ((int64_t)t * 64 + lane) * VE) = Vec16<T>::pack(f);
        };
        constexpr int NTASK = NQG + NKG + (BWD ? NKG : 0);
        for (int task = wave; task < NTASK; task += NW) {
            if (task < NQG) {
                if (BWD) row_group(sK, false, gksr, task);
                else row_group(sQ, true, gqs, task);
            } else if (task < NQG + NKG) {
                col_group(sK, false, gks, task - NQG);
            } else {
                col_group(sQ, true, gqs, task - NQG - NKG);
            }
        }
        // the state pass needs only the chunk's last row of the per-key
        // cumulative gate (the decay of the carried state); the backward
        // takes the whole gate, of either kind
        float* gg = a.ws.gcum + blk * C * (PK ? K : 1);
        if (PK && BWD) {
            for (int i = tid; i < C * K; i += NT) gg[i] = sG[(i / K) * LDG + i % K];
        } else if (PK) {
            for (int i = tid; i < K; i += NT) gg[(C - 1) * K + i] = sG[(C - 1) * LDG + i];
        } else {
            for (int i = tid; i < C; i += NT) gg[i] = sG[i];
        }
    }

    // ---- a2: beta-scaled decay-masked strictly-lower K K^T -> sA (fp32), and
    // Aqk^T = K Q^T masked -> Aqk rows in HBM (lane: 4 consecutive columns)
    T* gaqk = static_cast<T*>(a.ws.aqk) + blk * C * C;
    if (!PK) {
        // waves 0..NB-1: K K^T row block I = wave, all NB column blocks (the
        // upper ones come out masked to zero); waves NB..2NB-1: Aqk^T for
        // the columns of token block I = wave - NB.  Every operand fragment
        // is loaded before the first product.
        static_assert(2 * NB <= NW, "one row block per wave");
        constexpr int NKS = K / KS;
        if (wave < 2 * NB) {
            const bool isq = wave >= NB;
            const int I = isq ? wave - NB : wave;
            // shared operand: K rows of block I (K K^T, as A) or Q rows of block I (Aqk^T, as B)
            const T* sh = (isq ? sQ : sK) + (16 * I + (lane & 15)) * LDK;
            typename M::frag fs[NKS], fo[NB][NKS];
#pragma unroll
            for (int s = 0; s < NKS; ++s) fs[s] = M::load(sh + s * KS, lane);
#pragma unroll
            for (int J = 0; J < NB; ++J)
#pragma unroll
                for (int s = 0; s < NKS; ++s)
                    fo[J][s] = M::load(sK + (16 * J + (lane & 15)) * LDK + s * KS, lane);
            f32x4 acc[NB];
#pragma unroll
            for (int J = 0; J < NB; ++J) acc[J] = zero4();
            if (!isq) {
#pragma unroll
                for (int J = 0; J < NB; ++J)
#pragma unroll
                    for (int s = 0; s < NKS; ++s) acc[J] = M::mma(fs[s], fo[J][s], acc[J]);
                // rows i = 16I + 4(l/16) + e, columns j = 16J + l%16
                float gi[4], bi[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    gi[e] = sG[16 * I + acc_row(lane, e)];
                    bi[e] = sB[16 * I + acc_row(lane, e)];
                }
#pragma unroll
                for (int J = 0; J < NB; ++J) {
                    const int j = 16 * J + acc_col(lane);
                    const float gj = sG[j];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = 16 * I + acc_row(lane, e);
                        const float x = bi[e] * exp2_hw(fminf(gi[e] - gj, 0.f)) * acc[J][e];
                        sA[i * LDA + j] = j < i ? x : 0.f;
                    }
                }
            } else if (!BWD) {
#pragma unroll
                for (int J = 0; J < NB; ++J)
#pragma unroll
                    for (int s = 0; s < NKS; ++s) acc[J] = M::mma(fo[J][s], fs[s], acc[J]);
                // Aqk^T tiles: rows j = 16J + 4(l/16) + e, column i = 16I + l%16
                const int i = 16 * I + acc_col(lane);
                const float gi = sG[i];
#pragma unroll
                for (int J = 0; J < NB; ++J) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int j = 16 * J + acc_row(lane, e);
                        const float x = a.scale * exp2_hw(fminf(gi - sG[j], 0.f)) * acc[J][e];
                        acc[J][e] = j <= i ? x : 0.f;
                    }
                    store4_frag(gaqk, i, 16 * J + 4 * (lane >> 4), C, acc[J]);
                }
            } else {
                // backward mode: Aqk tiles (rows i = 16I + 4(l/16) + e, column
                // j = 16J + l%16), stored as 4 consecutive columns of Aqk^T
#pragma unroll
                for (int J = 0; J < NB; ++J)
#pragma unroll
                    for (int s = 0; s < NKS; ++s) acc[J] = M::mma(fs[s], fo[J][s], acc[J]);
#pragma unroll
                for (int J = 0; J < NB; ++J) {
                    const int j = 16 * J + acc_col(lane);
                    const float gj = sG[j];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = 16 * I + acc_row(lane, e);
                        const float x = a.scale * exp2_hw(fminf(sG[i] - gj, 0.f)) * acc[J][e];
                        acc[J][e] = j <= i ? x : 0.f;
                    }
                    store4_frag(gaqk, j, 16 * I + 4 * (lane >> 4), C, acc[J]);
                }
            }
        }
    } else {
        // Off-diagonal block rows I = 1 .. NB-1, then the diagonal blocks'
        // quadrants, each from decay-scaled operands built in a scratch
        // buffer.  Two buffers alternate: while the products of round I read
        // one, the operands of the next round are built in the other, so
        // the waves without a tile of round I go on building and one barrier
        // separates the rounds.
        T* const sS0 = reinterpret_cast<T*>(smem + L::o_S);
        T* const sS1 = sS0 + L::SCR_ROWS * LDK;
        auto buf = [&](int I) { return (I & 1) ? sS0 : sS1; };   // round NB: the quadrants
        auto build_offdiag = [&](int I) {
            const int b = 16 * I;
            T* sS = buf(I);
            // rows [0,16): K_I 2^{G_I - G_b}; [16,32): Q_I 2^{G_I - G_b};
            // [32, 32 + b): K_J 2^{G_b - G_J} for all J < I
            for (int i = tid; i < (32 + b) * (K / EV); i += NT) {   // one 16-byte vector each
                const int r = i / (K / EV), d0 = (i - r * (K / EV)) * EV;
                const bool later = r < 32;   // rows of block I (scaled to b) or of J < I (from b)
                const int tok = later ? b + (r & 15) : r - 32;
                const uint4 xv = *reinterpret_cast<const uint4*>((later && r >= 16 ? sQ : sK) + tok * LDK + d0);
                float f[EV];
#pragma unroll
                for (int e4 = 0; e4 < EV; e4 += 4) {
                    const float4 gt = *reinterpret_cast<const float4*>(sG + tok * LDG + d0 + e4);
                    const float4 gb = *reinterpret_cast<const float4*>(sG + b * LDG + d0 + e4);
                    const float dt[4] = {gt.x - gb.x, gt.y - gb.y, gt.z - gb.z, gt.w - gb.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        f[e4 + e] = Vec16<T>::get(xv, e4 + e) * exp2_hw(fminf(later ? dt[e] : -dt[e], 0.f));
                }
                *reinterpret_cast<uint4*>(sS + r * LDK + d0) = Vec16<T>::pack(f);
            }
        };
        auto tiles_offdiag = [&](int I) {
            const T* sS = buf(I);
            for (int job = wave; job < 2 * I; job += NW) {
                const bool isq = job >= I;
                const int J = isq ? job - I : job;
                if (!isq) {
                    f32x4 acc = mma_tile<T>(sS, LDK, sS + (32 + 16 * J) * LDK, LDK, K, lane,
                                            zero4());
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = 16 * I + acc_row(lane, e), j = 16 * J + acc_col(lane);
                        sA[i * LDA + j] = sB[i] * acc[e];
                    }
                } else if (!BWD) {
                    // Aqk^T tile: rows j (block J), columns i (block I)
                    f32x4 acc = mma_tile<T>(sS + (32 + 16 * J) * LDK, LDK, sS + 16 * LDK, LDK, K,
                                            lane, zero4());
                    acc *= a.scale;
                    store4_frag(gaqk, 16 * I + acc_col(lane), 16 * J + 4 * (lane >> 4), C, acc);
                } else {
                    // backward mode: the Aqk tile (rows i, columns j), stored
                    // as 4 consecutive columns of Aqk^T
                    f32x4 acc = mma_tile<T>(sS + 16 * LDK, LDK, sS + (32 + 16 * J) * LDK, LDK, K,
                                            lane, zero4());
                    acc *= a.scale;
                    store4_frag(gaqk, 16 * J + acc_col(lane), 16 * I + 4 * (lane >> 4), C, acc);
                }
            }
        };
        // lower-left 8x8 quadrant of each diagonal block, with b = 16 I + 8:
        // rows [0, C/2): the 8 later K rows of each block, K 2^{G - G_b};
        // [C/2, C): the same Q rows; [C, 3C/2): the 8 earlier K rows,
        // K 2^{G_b - G}.  One 16x16 tile covers two blocks; its two
        // cross-block quadrants are dropped.
        auto build_quadrants = [&]() {
            T* sS = buf(NB);
            for (int i = tid; i < (3 * C / 2) * (K / EV); i += NT) {
                const int r = i / (K / EV), d0 = (i - r * (K / EV)) * EV;
                const int set = r / (C / 2), rr = r - set * (C / 2), Ib = rr / 8;
                const int b = 16 * Ib + 8, tok = set < 2 ? b + (rr & 7) : 16 * Ib + (rr & 7);
                const uint4 xv = *reinterpret_cast<const uint4*>((set == 1 ? sQ : sK) + tok * LDK + d0);
                float f[EV];
#pragma unroll
                for (int e4 = 0; e4 < EV; e4 += 4) {
                    const float4 gt = *reinterpret_cast<const float4*>(sG + tok * LDG + d0 + e4);
                    const float4 gb = *reinterpret_cast<const float4*>(sG + b * LDG + d0 + e4);
                    const float dt[4] = {gt.x - gb.x, gt.y - gb.y, gt.z - gb.z, gt.w - gb.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        f[e4 + e] = Vec16<T>::get(xv, e4 + e) * exp2_hw(fminf(set < 2 ? dt[e] : -dt[e], 0.f));
                }
                *reinterpret_cast<uint4*>(sS + r * LDK + d0) = Vec16<T>::pack(f);
            }
        };
        static_assert(NB % 2 == 0, "diagonal blocks in pairs");
        build_offdiag(1);
        __syncthreads();
        for (int I = 1; I < NB; ++I) {
            tiles_offdiag(I);
            if (I + 1 < NB)
                build_offdiag(I + 1);
            else
                build_quadrants();
            __syncthreads();
        }
        const T* sS = buf(NB);
        if (wave >= NB && wave < 2 * NB) {   // job (pair P of blocks, A or Aqk); waves
                                             // 0..NB-1 take the triangles meanwhile
            const int P = (wave - NB) % (NB / 2);
            const bool isq = wave - NB >= NB / 2;
            const int g4 = lane >> 4;
            if (!isq) {
                // rows: later K of blocks 2P, 2P+1; columns: their earlier K
                const f32x4 acc = mma_tile<T>(sS + 16 * P * LDK, LDK, sS + (C + 16 * P) * LDK, LDK, K,
                                              lane, zero4());
                const int cc = acc_col(lane);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int rr = acc_row(lane, e);
                    if (rr / 8 == cc / 8) {
                        const int Ib = 2 * P + rr / 8, i = 16 * Ib + 8 + (rr & 7), j = 16 * Ib + (cc & 7);
                        sA[i * LDA + j] = sB[i] * acc[e];
                    }
                }
            } else if (!BWD) {
                // Aqk^T: rows the earlier K (j), columns the later Q (i)
                f32x4 acc = mma_tile<T>(sS + (C + 16 * P) * LDK, LDK, sS + (C / 2 + 16 * P) * LDK, LDK,
                                        K, lane, zero4());
                const int cc = acc_col(lane);
                if (g4 / 2 == cc / 8) {   // rows 4 g4 .. 4 g4 + 3 lie in column cc's block
                    const int Ib = 2 * P + cc / 8;
                    acc *= a.scale;
                    store4_frag(gaqk, 16 * Ib + 8 + (cc & 7), 16 * Ib + 4 * (g4 & 1), C, acc);
                }
            } else {
                // backward mode, Aqk: rows the later Q (i), columns the
                // earlier K (j); 4 consecutive columns of Aqk^T per lane
                f32x4 acc = mma_tile<T>(sS + (C / 2 + 16 * P) * LDK, LDK, sS + (C + 16 * P) * LDK, LDK,
                                        K, lane, zero4());
                const int cc = acc_col(lane);
                if (g4 / 2 == cc / 8) {
                    const int Ib = 2 * P + cc / 8;
                    acc *= a.scale;
                    store4_frag(gaqk, 16 * Ib + (cc & 7), 16 * Ib + 8 + 4 * (g4 & 1), C, acc);
                }
            }
        }
        // zeros of Aqk's strict upper triangle (Aqk^T's lower one in the
        // backward mode), by the waves of the quadrant jobs: every 8-column
        // piece of a row that lies wholly on the zero side; the pieces the
        // diagonal crosses are written whole by the triangles below.  (A's
        // upper triangle is never read: the substitution reads below the
        // diagonal only, and Ainv's upper blocks are masked.)
        if (wave >= NB) {
            if constexpr (sizeof(T) == 2) {   // a piece is one 16-byte group of the fragment order
                for (int pc = tid - 64 * NB; pc < C * C / 8; pc += NT - 64 * NB) {
                    const int r = pc >> 3, p8 = 8 * (pc & 7);
                    if (BWD ? p8 + 7 < r : p8 > r)
                        *reinterpret_cast<uint4*>(gaqk + FragOrder<T>::off(r, p8, C)) = uint4{0u, 0u, 0u, 0u};
                }
            } else {
                for (int i = tid - 64 * NB; i < C * C; i += NT - 64 * NB) {
                    const int r = i / C, j = i - r * C;
                    if ((BWD ? j < r : j > r) && (j >> 3) != (r >> 3))
                        Elem<T>::store(gaqk + FragOrder<T>::off(r, j, C), 0.f);
                }
            }
        }
        // the two 8x8 triangles of each diagonal block (pairs j <= i inside
        // one 8-token half), wave I taking block I: lane (token t of the
        // block, channel quarter cq) holds its token's key, query and gate
        // for CQ channels.  Offset O pairs token t with j = t - O: K_j comes
        // from lane t - O by a row shift (DPP, inside the 16-lane row of one
        // channel quarter), and 2^{G_t - G_j} per channel is the running
        // product E(O) = E(O-1) alpha_{t-O+1} of the gate factors
        // alpha_s = 2^{G_s - G_{s-1}} <= 1 (a row shift of O-1 away), so no
        // exponential is taken per pair and nothing overflows.  Offsets past
        // the half's first token (O > t % 8) are computed and dropped.  The
        // quarters' sums meet by row swaps, after which every lane holds
        // them all: lane (t, cq) writes A for offsets 2cq, 2cq + 1 and two
        // of the eight entries of the 8-column piece of Aqk (or Aqk^T) that
        // holds its token's row of the half, zeros included.
        if (wave < NB) {
            constexpr int CQ = K / 4;
            static_assert(CQ % EV == 0 && CQ % 4 == 0, "whole vectors per lane");
            const int I = wave, t = lane & 15, cq = lane >> 4, i = 16 * I + t, c0 = CQ * cq;
            auto shr = [](float x, auto o) {   // the value of lane t - o of the row, 0 outside
                return __int_as_float(
                    __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + decltype(o)::value, 0xf, 0xf, true));
            };
            auto shl = [](float x, auto o) {   // the value of lane t + o of the row, 0 outside
                return __int_as_float(
                    __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x100 + decltype(o)::value, 0xf, 0xf, true));
            };
            // the sum over the wave's four rows (channel quarters), in every lane
            auto rows_sum = [](float x) {
                const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
                const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
                const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
                return __uint_as_float(b[0]) + __uint_as_float(b[1]);
            };
            float kf[CQ], qf[CQ], al[CQ], E[CQ];
#pragma unroll
            for (int v = 0; v < CQ / EV; ++v) {
                const uint4 xk = *reinterpret_cast<const uint4*>(sK + i * LDK + c0 + v * EV);
                const uint4 xq = *reinterpret_cast<const uint4*>(sQ + i * LDK + c0 + v * EV);
#pragma unroll
                for (int e = 0; e < EV; ++e) {
                    kf[v * EV + e] = Vec16<T>::get(xk, e);
                    qf[v * EV + e] = Vec16<T>::get(xq, e);
                }
            }
#pragma unroll
            for (int v = 0; v < CQ / 4; ++v) {
                const float4 x = *reinterpret_cast<const float4*>(sG + i * LDG + c0 + 4 * v);
                const float gx[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    al[4 * v + e] = exp2_hw(fminf(gx[e] - shr(gx[e], std::integral_constant<int, 1>()), 0.f));
            }
            float akk[8], aqk[8];
            auto offset = [&](auto oc) {
                constexpr int O = decltype(oc)::value;
                float sk0 = 0.f, sk1 = 0.f, sq0 = 0.f, sq1 = 0.f;
#pragma unroll
                for (int c = 0; c < CQ; ++c) {
                    float kj;
                    if constexpr (O == 0) {
                        kj = kf[c];
                    } else {
                        if constexpr (O == 1) E[c] = al[c];
                        else E[c] *= shr(al[c], std::integral_constant<int, O - 1>());
                        kj = shr(kf[c], std::integral_constant<int, O>()) * E[c];
                    }
                    if (c & 1) {
                        sk1 += kf[c] * kj;
                        sq1 += qf[c] * kj;
                    } else {
                        sk0 += kf[c] * kj;
                        sq0 += qf[c] * kj;
                    }
                }
                akk[O] = sk0 + sk1;
                aqk[O] = sq0 + sq1;
                // keep the offsets in order: left alone, the compiler hoists
                // the row shifts of later offsets and keeps them all live
                asm volatile("" : "+v"(akk[O]), "+v"(aqk[O]));
#pragma unroll
                for (int c = 0; c < CQ; ++c) asm volatile("" : "+v"(E[c]));
            };
            offset(std::integral_constant<int, 0>());
            offset(std::integral_constant<int, 1>());
            offset(std::integral_constant<int, 2>());
            offset(std::integral_constant<int, 3>());
            offset(std::integral_constant<int, 4>());
            offset(std::integral_constant<int, 5>());
            offset(std::integral_constant<int, 6>());
            offset(std::integral_constant<int, 7>());
#pragma unroll
            for (int O = 0; O < 8; ++O) {
                akk[O] = rows_sum(akk[O]);
                aqk[O] = rows_sum(aqk[O]) * a.scale;
            }
            // the pairs of the stored row: (token t, t - O) in the forward
            // mode; (t + O, t) in the backward mode, whose row is a column
            // of Aqk (a row shift of O brings pair (t + O, t) to lane t)
            float pv[8];
            pv[0] = aqk[0];
            if constexpr (BWD) {
                pv[1] = shl(aqk[1], std::integral_constant<int, 1>());
                pv[2] = shl(aqk[2], std::integral_constant<int, 2>());
                pv[3] = shl(aqk[3], std::integral_constant<int, 3>());
                pv[4] = shl(aqk[4], std::integral_constant<int, 4>());
                pv[5] = shl(aqk[5], std::integral_constant<int, 5>());
                pv[6] = shl(aqk[6], std::integral_constant<int, 6>());
                pv[7] = shl(aqk[7], std::integral_constant<int, 7>());
            } else {
#pragma unroll
                for (int O = 1; O < 8; ++O) pv[O] = aqk[O];
            }
            const int tt = t & 7;
            float ev[2], av[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int e = 2 * cq + u;        // column 8(t/8) + e of the piece
                const int O = BWD ? e - tt : tt - e;
                float x = 0.f, y = 0.f;
#pragma unroll
                for (int o = 0; o < 8; ++o) {
                    x = o == O ? pv[o] : x;
                    y = o == e ? akk[o] : y;
                }
                ev[u] = x;
                av[u] = y;
            }
            // A: offsets 2cq, 2cq + 1 of token t (j = i - O > the half's start - 1)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int O = 2 * cq + u;
                if (O > 0 && O <= tt) sA[i * LDA + i - O] = sB[i] * av[u];
            }
            // Aqk: entries 2cq, 2cq + 1 of the piece (4 bytes)
            const int col = 16 * I + 8 * (t >> 3) + 2 * cq;
            if constexpr (sizeof(T) == 2) {
                *reinterpret_cast<uint32_t*>(gaqk + FragOrder<T>::off(i, col, C)) = pack_bf16x2(ev[0], ev[1]);
            } else {
                Elem<T>::store(gaqk + FragOrder<T>::off(i, col, C), ev[0]);
                Elem<T>::store(gaqk + FragOrder<T>::off(i, col + 1, C), ev[1]);
            }
        }
    }
    __syncthreads();

    // ---- a3: Ainv = (I + A)^{-1}
    // diagonal blocks: wave w inverts block w by forward substitution; lane
    // c < 16 computes column c
    if (wave < NB && lane < 16) {
        float* blkA = sA + 16 * wave * LDA + 16 * wave;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = (r == lane) ? 1.f : 0.f;
        // right-looking: once x[m] is final it is taken out of every later
        // row, so the dependent chain is 16 steps long rather than 120 (each
        // x[r] still subtracts its terms in the order m = 0, 1, ...)
#pragma unroll
        for (int m = 0; m < 16; ++m)
#pragma unroll
            for (int r = m + 1; r < 16; ++r) x[r] -= blkA[r * LDA + m] * x[m];
        // the block is only touched by this wave, whose LDS accesses stay in order
#pragma unroll
        for (int r = 0; r < 16; ++r) blkA[r * LDA + lane] = x[r];
    }
    __syncthreads();
    // off-diagonal blocks, one block row at a time
    for (int I = 1; I < NB; ++I) {
        f32x4 x = zero4();
        if (wave < I) {
            const int J = wave;
            f32x4 p = zero4();
            for (int m = J; m < I; ++m)
                p = mma_f32_rr(sA + 16 * I * LDA + 16 * m, LDA, sA + 16 * m * LDA + 16 * J, LDA, 16,
                               lane, p);
            float* pw = sP + wave * 16 * 17;
#pragma unroll
            for (int e = 0; e < 4; ++e) pw[acc_row(lane, e) * 17 + acc_col(lane)] = p[e];
            // same wave wrote pw: the LDS writes are ordered before its reads
            __builtin_amdgcn_s_waitcnt(0);
            __builtin_amdgcn_wave_barrier();
            x = mma_f32_rr(sA + 16 * I * LDA + 16 * I, LDA, pw, 17, 16, lane, zero4());
        }
        __syncthreads();   // every wave is done reading block row I of A
        if (wave < I) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sA[(16 * I + acc_row(lane, e)) * LDA + 16 * wave + acc_col(lane)] = -x[e];
        }
        __syncthreads();
    }

    // ---- Ainv with its columns scaled: A1 = Ainv diag(beta gamma) (for W),
    // A2 = Ainv diag(beta) (for U).  Per-key gate: gamma is per channel and
    // goes into K instead, so W uses A2 too.  Upper blocks were never
    // written and are taken as zero.
    {
        static_assert(C * C == NT * 8, "one 8-column slice per thread");
        const int r = tid / (C / 8), j0 = (tid % (C / 8)) * 8;
        const bool up = j0 / 16 > r / 16;
        float4 x0 = *reinterpret_cast<const float4*>(sA + r * LDA + j0);
        float4 x1 = *reinterpret_cast<const float4*>(sA + r * LDA + j0 + 4);
        if (up) x0 = x1 = make_float4(0.f, 0.f, 0.f, 0.f);
        const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        if (STORE_AINV && !BWD) {
            float* gai = a.ws.ainv + blk * C * C + r * C + j0;
            *reinterpret_cast<float4*>(gai) = x0;
            *reinterpret_cast<float4*>(gai + 4) = x1;
        }
        if (BWD) {   // the backward takes it as an MFMA operand: element type, row-major
            T* gai = reinterpret_cast<T*>(a.ws.ainv) + blk * C * C + r * C + j0;
#pragma unroll
            for (int e = 0; e < 8; e += EV) *reinterpret_cast<uint4*>(gai + e) = Vec16<T>::pack(x + e);
        }
        float y1[8], y2[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int j = j0 + e;
            y2[e] = x[e] * sB[j];
            y1[e] = PK ? y2[e] : y2[e] * sE[j];
        }
        __syncthreads();   // everyone has read sA before it is overwritten
#pragma unroll
        for (int e = 0; e < 8; e += EV) {
            *reinterpret_cast<uint4*>(sA1 + r * LDC + j0 + e) = Vec16<T>::pack(y1 + e);
            *reinterpret_cast<uint4*>(sA2 + r * LDC + j0 + e) = Vec16<T>::pack(y2 + e);
        }
    }
    // per-key gate: K 2^{G} (row-major) for W, in the scratch region
    const T* sKW = sK;
    const T* sAW = sA1;
    if (PK) {
        T* sKg = reinterpret_cast<T*>(smem + L::o_S);
#pragma unroll
        for (int p = 0; p < PKQ; ++p) {
            const int i = tid + NT * p, r = i / (K / EV), d0 = (i % (K / EV)) * EV;
            if (i < NKV) {
                const uint4 xk = *reinterpret_cast<const uint4*>(sK + r * LDK + d0);
                float f[EV];
#pragma unroll
                for (int e = 0; e < EV; ++e) f[e] = exp2_hw(sG[r * LDG + d0 + e]) * Vec16<T>::get(xk, e);
                *reinterpret_cast<uint4*>(sKg + r * LDK + d0) = Vec16<T>::pack(f);
            }
        }
        sKW = sKg;
        sAW = sA2;
    }
    __syncthreads();

    // ---- a4: W^T = K^T A1^T and U = A2 V.  Wave w takes token block
    // I = w % NB and every (NW/NB)-th column block D of K and of V; the A1 / A2
    // rows of block I are loaded once and shared by all its tiles.
    {
        static_assert(NW % NB == 0 && (K / 16) % (NW / NB) == 0 && (V / 16) % (NW / NB) == 0,
                      "column blocks split evenly over the waves of a token block");
        constexpr int G = NW / NB, WD = (K / 16) / G, UD = (V / 16) / G, NKM = C / KS;
        T* gw = static_cast<T*>(a.ws.w) + blk * C * K;
        T* gu = static_cast<T*>(a.ws.u) + blk * C * V;
        const int I = wave % NB, d0 = wave / NB;
        const int kn = min(C, ((16 * (I + 1) + KS - 1) / KS) * KS);
        const T* bw = sAW + (16 * I + (lane & 15)) * LDC;
        const T* bu = sA2 + (16 * I + (lane & 15)) * LDC;
        typename M::frag fw[NKM], fu[NKM];
#pragma unroll
        for (int s = 0; s < NKM; ++s)
            if (s * KS < kn) {
                fw[s] = M::load(bw + s * KS, lane);
                fu[s] = M::load(bu + s * KS, lane);
            }
        f32x4 aw[WD], au[UD];
#pragma unroll
        for (int m = 0; m < WD; ++m) {
            const int D = d0 + G * m;
            aw[m] = zero4();
#pragma unroll
            for (int s = 0; s < NKM; ++s)
                if (s * KS < kn)
                    aw[m] = M::mma(M::load_t(sKW + s * KS * LDK + 16 * D, LDK, lane), fw[s], aw[m]);
        }
#pragma unroll
        for (int m = 0; m < UD; ++m) {
            const int D = d0 + G * m;
            au[m] = zero4();
#pragma unroll
            for (int s = 0; s < NKM; ++s)
                if (s * KS < kn)
                    au[m] = M::mma(fu[s], M::load_t(sV + s * KS * LDV + 16 * D, LDV, lane), au[m]);
        }
        // W^T tiles: lane holds W[i][4 consecutive d] -> fragment order;
        // U tiles: lane holds U[4 consecutive i][d] -> accumulator order
        const int i = 16 * I + acc_col(lane);
#pragma unroll
        for (int m = 0; m < WD; ++m)
            store4_frag(gw, i, 16 * (d0 + G * m) + 4 * (lane >> 4), K, aw[m]);
        if (BWD) {   // W^T in fragment order as well (rows = keys): W tiles,
                     // 4 consecutive tokens of one key per lane
            T* gwt = static_cast<T*>(a.ws.wt) + blk * C * K;
#pragma unroll
            for (int m = 0; m < WD; ++m) {
                const int D = d0 + G * m;
                f32x4 wn = zero4();
#pragma unroll
                for (int s = 0; s < NKM; ++s)
                    if (s * KS < kn)
                        wn = M::mma(fw[s], M::load_t(sKW + s * KS * LDK + 16 * D, LDK, lane), wn);
                store4_frag(gwt, 16 * D + acc_col(lane), 16 * I + 4 * (lane >> 4), C, wn);
            }
        }
#pragma unroll
        for (int m = 0; m < UD; ++m)
            store4(gu + acc_order_off(16 * I + acc_row(lane, 0), 16 * (d0 + G * m) + acc_col(lane), V),
                   au[m]);
    }
}

template <typename T, int K, int V, int C, bool PK>
static hipError_t launch_intra_t(const IntraLaunch& a) {
    dim3 grid((unsigned)(a.map.max_chunks * a.H));
    if (a.bwd) {
        if (!a.ws.ainv || !a.ws.ksr || !a.ws.wt) return hipErrorInvalidValue;
        hipLaunchKernelGGL((intra_kernel<T, K, V, C, PK, true, true>), grid, dim3(INTRA_THREADS), 0,
                           a.stream, a);
        return hipGetLastError();
    }
    if (a.ws.ainv)
        hipLaunchKernelGGL((intra_kernel<T, K, V, C, PK, true>), grid, dim3(INTRA_THREADS), 0,
                           a.stream, a);
    else
        hipLaunchKernelGGL((intra_kernel<T, K, V, C, PK, false>), grid, dim3(INTRA_THREADS), 0,
                           a.stream, a);
    return hipGetLastError();
}

template <typename T, int C>
static hipError_t launch_intra_c(const IntraLaunch& a) {
#define GDN_INTRA_CASE(KK, VV)                                                   \
    if (a.K == KK && a.V == VV)                                                  \
        return a.per_key ? launch_intra_t<T, KK, VV, C, true>(a)                 \
                         : launch_intra_t<T, KK, VV, C, false>(a);
    GDN_INTRA_CASE(64, 64)
    GDN_INTRA_CASE(64, 128)
#undef GDN_INTRA_CASE
    // with K = 128 the fp32 per-key variant exceeds the 160 KB of LDS
    if (a.K == 128 && a.V == 64) {
        if (!a.per_key) return launch_intra_t<T, 128, 64, C, false>(a);
        if constexpr (sizeof(T) == 2) return launch_intra_t<T, 128, 64, C, true>(a);
        return hipErrorInvalidValue;
    }
    if (a.K == 128 && a.V == 128) {
        if (!a.per_key) return launch_intra_t<T, 128, 128, C, false>(a);
        if constexpr (sizeof(T) == 2) return launch_intra_t<T, 128, 128, C, true>(a);
        return hipErrorInvalidValue;
    }
    return hipErrorInvalidValue;
}

hipError_t launch_intra(const IntraLaunch& a) {
    if (a.C != 64) return hipErrorInvalidValue;
    return a.bf16 ? launch_intra_c<bf16, 64>(a) : launch_intra_c<float, 64>(a);
}

}  // namespace gdn
