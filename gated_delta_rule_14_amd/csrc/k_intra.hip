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
// exponents <= 0, so they run on MFMA without overflow; the diagonal blocks
// are summed pair by pair.  gamma and gamma_C/gamma become per-channel.
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
    static constexpr int NB = C / 16;
    static constexpr int SCR_ROWS = 32 + C - 16;   // per-key scaled operands (>= C)
    static constexpr size_t o_K = 0;
    static constexpr size_t o_Q = o_K + sizeof(T) * C * LDK;
    static constexpr size_t o_V = o_Q + sizeof(T) * C * LDK;
    static constexpr size_t o_A = o_V + sizeof(T) * C * LDV;
    static constexpr size_t o_G = o_A + sizeof(float) * C * LDA;
    static constexpr size_t o_B = o_G + sizeof(float) * C * (PK ? K : 1);
    static constexpr size_t o_E = o_B + sizeof(float) * C;     // 2^{G_r}
    static constexpr size_t o_F = o_E + sizeof(float) * C;     // 2^{G_C-1 - G_r}
    static constexpr size_t o_P = o_F + sizeof(float) * C;
    static constexpr size_t o_S = o_P + sizeof(float) * 4 * 16 * 17;
    static constexpr size_t bytes = o_S + (PK ? sizeof(T) * SCR_ROWS * LDK : 0);
    // Ainv diag(beta gamma) goes where Q was, Ainv diag(beta) where A was
    static_assert(C * LDC * sizeof(T) <= C * LDK * sizeof(T), "A1 fits the Q region");
    static_assert(C * LDC * sizeof(T) <= C * LDA * sizeof(float), "A2 fits the A region");
};

template <typename T, int K, int V, int C, bool PK, bool STORE_AINV>
__global__ __launch_bounds__(INTRA_THREADS) void intra_kernel(IntraLaunch a) {
    typedef IntraSmem<T, K, V, C, PK> L;
    typedef Mma<T> M;
    constexpr int NT = INTRA_THREADS, NW = NT / 64;
    constexpr int LDK = L::LDK, LDV = L::LDV, LDC = L::LDC, LDA = L::LDA, NB = L::NB;
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

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t c = blockIdx.x, h = blockIdx.y, H = a.H;

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

    // ---- loads: K, Q, V rows (zeros past n), issued before any is used
    constexpr int NKV = C * K / EV, NVV = C * V / EV;
    constexpr int PKQ = (NKV + NT - 1) / NT, PV = (NVV + NT - 1) / NT;
    uint4 kr[PKQ], qr[PKQ], vr[PV];
#pragma unroll
    for (int p = 0; p < PKQ; ++p) {
        const int i = tid + NT * p, r = i / (K / EV), cv = i % (K / EV);
        kr[p] = qr[p] = make_uint4(0, 0, 0, 0);
        if (i < NKV && r < n) {
            kr[p] = *reinterpret_cast<const uint4*>(k + ((t0 + r) * H + h) * K + cv * EV);
            qr[p] = *reinterpret_cast<const uint4*>(q + ((t0 + r) * H + h) * K + cv * EV);
        }
    }
#pragma unroll
    for (int p = 0; p < PV; ++p) {
        const int i = tid + NT * p, r = i / (V / EV), cv = i % (V / EV);
        vr[p] = make_uint4(0, 0, 0, 0);
        if (i < NVV && r < n)
            vr[p] = *reinterpret_cast<const uint4*>(v + ((t0 + r) * H + h) * V + cv * EV);
    }

    // ---- a1: gates and beta; cumulative log2 gate (rows >= n: g = 0, beta = 0)
    if (!PK) {
        if (wave == 0) {
            const int r = lane;
            float gl = 0.f, bt = 0.f;
            if (r < n) {
                gl = a.g[(t0 + r) * H + h] * LOG2E;
                bt = a.beta[(t0 + r) * H + h];
            }
            const float G = wave_incl_scan(gl, lane);
            const float Gc = __shfl(G, C - 1, 64);
            if (r < C) {
                sG[r] = G;
                sB[r] = bt;
                sE[r] = exp2f(G);
                sF[r] = exp2f(fminf(Gc - G, 0.f));
            }
        }
    } else {
        for (int d = tid; d < K; d += NT) {
            float acc = 0.f;
            float gv[16];
            for (int r0 = 0; r0 < C; r0 += 16) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int r = r0 + i;
                    gv[i] = r < n ? a.g[((t0 + r) * H + h) * K + d] * LOG2E : 0.f;
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    acc += gv[i];
                    sG[(r0 + i) * K + d] = acc;
                }
            }
        }
        for (int r = tid; r < C; r += NT) sB[r] = r < n ? a.beta[(t0 + r) * H + h] : 0.f;
    }
#pragma unroll
    for (int p = 0; p < PKQ; ++p) {
        const int i = tid + NT * p, r = i / (K / EV), cv = i % (K / EV);
        if (i < NKV) {
            *reinterpret_cast<uint4*>(sK + r * LDK + cv * EV) = kr[p];
            *reinterpret_cast<uint4*>(sQ + r * LDK + cv * EV) = qr[p];
        }
    }
#pragma unroll
    for (int p = 0; p < PV; ++p) {
        const int i = tid + NT * p, r = i / (V / EV), cv = i % (V / EV);
        if (i < NVV) *reinterpret_cast<uint4*>(sV + r * LDV + cv * EV) = vr[p];
    }
    __syncthreads();

    // ---- outputs that need only G, Q, K (stored straight from registers):
    // Qs = scale 2^{G} Q, Ks = 2^{G_C - G} K, and the cumulative gate
    {
        T* gqs = static_cast<T*>(a.ws.qs) + blk * C * K;
        T* gks = static_cast<T*>(a.ws.ks) + blk * C * K;
#pragma unroll
        for (int p = 0; p < PKQ; ++p) {
            const int i = tid + NT * p, r = i / (K / EV), d0 = (i % (K / EV)) * EV;
            if (i < NKV) {
                const uint4 xq = *reinterpret_cast<const uint4*>(sQ + r * LDK + d0);
                const uint4 xk = *reinterpret_cast<const uint4*>(sK + r * LDK + d0);
                float fq[EV], fk[EV];
                if (!PK) {
                    const float eq = a.scale * sE[r], ek = sF[r];
#pragma unroll
                    for (int e = 0; e < EV; ++e) {
                        fq[e] = eq * Vec16<T>::get(xq, e);
                        fk[e] = ek * Vec16<T>::get(xk, e);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < EV; ++e) {
                        const float gr = sG[r * K + d0 + e], gc = sG[(C - 1) * K + d0 + e];
                        fq[e] = a.scale * exp2f(gr) * Vec16<T>::get(xq, e);
                        fk[e] = exp2f(fminf(gc - gr, 0.f)) * Vec16<T>::get(xk, e);
                    }
                }
                *reinterpret_cast<uint4*>(gqs + r * K + d0) = Vec16<T>::pack(fq);
                *reinterpret_cast<uint4*>(gks + r * K + d0) = Vec16<T>::pack(fk);
            }
        }
        float* gg = a.ws.gcum + blk * C * (PK ? K : 1);
        for (int i = tid; i < C * (PK ? K : 1); i += NT) gg[i] = sG[i];
    }

    // ---- a2: beta-scaled decay-masked strictly-lower K K^T -> sA (fp32), and
    // Aqk^T = K Q^T masked -> Aqk rows in HBM (lane: 4 consecutive columns)
    T* gaqk = static_cast<T*>(a.ws.aqk) + blk * C * C;
    if (!PK) {
        constexpr int NT2 = NB * (NB + 1) / 2, NZ = NB * (NB - 1) / 2;
        for (int job = wave; job < 2 * NT2 + NZ; job += NW) {
            if (job < 2 * NT2) {
                const bool isq = job >= NT2;
                int t = isq ? job - NT2 : job, I = 0;
                while (t > I) { t -= I + 1; ++I; }
                const int J = t;
                // K K^T tile (I, J): rows i in block I, columns j in block J.
                // Q K^T as its transpose: rows j (block J, from K), columns i (block I, from Q)
                const T* A0 = sK + 16 * (isq ? J : I) * LDK;
                const T* B0 = (isq ? sQ : sK) + 16 * (isq ? I : J) * LDK;
                f32x4 acc = mma_tile<T>(A0, LDK, B0, LDK, K, lane, zero4());
                if (!isq) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = 16 * I + acc_row(lane, e), j = 16 * J + acc_col(lane);
                        sA[i * LDA + j] = j < i ? sB[i] * exp2f(fminf(sG[i] - sG[j], 0.f)) * acc[e]
                                                : 0.f;
                    }
                } else {
                    const int i = 16 * I + acc_col(lane);
                    const float gi = sG[i];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int j = 16 * J + acc_row(lane, e);
                        acc[e] = j <= i ? a.scale * exp2f(fminf(gi - sG[j], 0.f)) * acc[e] : 0.f;
                    }
                    store4(gaqk + i * C + 16 * J + 4 * (lane >> 4), acc);
                }
            } else {
                // an upper block of Aqk: zeros
                int t = job - 2 * NT2, I = 0;
                while (t >= NB - 1 - I) { t -= NB - 1 - I; ++I; }
                const int J = I + 1 + t;
                store4(gaqk + (16 * I + acc_col(lane)) * C + 16 * J + 4 * (lane >> 4), zero4());
            }
        }
    } else {
        T* sS = reinterpret_cast<T*>(smem + L::o_S);
        for (int I = 1; I < NB; ++I) {
            const int b = 16 * I;
            __syncthreads();   // previous I's tiles have read the scratch
            // rows [0,16): K_I 2^{G_I - G_b}; [16,32): Q_I 2^{G_I - G_b};
            // [32, 32 + b): K_J 2^{G_b - G_J} for all J < I
            for (int i = tid; i < (32 + b) * K; i += NT) {
                const int r = i / K, d = i - r * K;
                float x;
                if (r < 32) {
                    const int tok = b + (r & 15);
                    const T* src = (r < 16 ? sK : sQ) + tok * LDK + d;
                    x = Elem<T>::load(src) * exp2f(fminf(sG[tok * K + d] - sG[b * K + d], 0.f));
                } else {
                    const int tok = r - 32;
                    x = Elem<T>::load(sK + tok * LDK + d) *
                        exp2f(fminf(sG[b * K + d] - sG[tok * K + d], 0.f));
                }
                Elem<T>::store(sS + r * LDK + d, x);
            }
            __syncthreads();
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
                } else {
                    // Aqk^T tile: rows j (block J), columns i (block I)
                    f32x4 acc = mma_tile<T>(sS + (32 + 16 * J) * LDK, LDK, sS + 16 * LDK, LDK, K,
                                            lane, zero4());
                    acc *= a.scale;
                    store4(gaqk + (16 * I + acc_col(lane)) * C + 16 * J + 4 * (lane >> 4), acc);
                }
            }
        }
        // upper blocks of Aqk: zeros (those of A are masked when Ainv is read)
        for (int i = tid; i < C * C; i += NT) {
            const int r = i / C, j = i - r * C;
            if (j / 16 > r / 16) Elem<T>::store(gaqk + i, 0.f);
        }
        // diagonal 16x16 blocks, pair by pair: thread = (block, row, slice of d)
        {
            constexpr int SL = NT / (NB * 16);      // threads per row
            constexpr int DQ = K / SL;
            const int I = tid / (16 * SL), i = 16 * I + (tid % (16 * SL)) / SL, s = tid % SL;
            for (int j = 16 * I; j < 16 * I + 16; ++j) {
                float akk = 0.f, aqk = 0.f;
                if (j <= i) {
                    for (int d = s * DQ; d < s * DQ + DQ; ++d) {
                        const float dec = exp2f(fminf(sG[i * K + d] - sG[j * K + d], 0.f));
                        const float kj = Elem<T>::load(sK + j * LDK + d) * dec;
                        akk += Elem<T>::load(sK + i * LDK + d) * kj;
                        aqk += Elem<T>::load(sQ + i * LDK + d) * kj;
                    }
                }
#pragma unroll
                for (int off = 1; off < SL; off <<= 1) {
                    akk += __shfl_xor(akk, off, 64);
                    aqk += __shfl_xor(aqk, off, 64);
                }
                if (s == 0) {
                    sA[i * LDA + j] = j < i ? sB[i] * akk : 0.f;
                    Elem<T>::store(gaqk + i * C + j, j <= i ? a.scale * aqk : 0.f);
                }
            }
        }
    }
    __syncthreads();

    // ---- a3: Ainv = (I + A)^{-1}
    // diagonal blocks: wave w inverts block w; lane c < 16 computes column c
    if (wave < NB && lane < 16) {
        float* blkA = sA + 16 * wave * LDA + 16 * wave;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = (r == lane) ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < r; ++m) acc -= blkA[r * LDA + m] * x[m];
            x[r] = acc;
        }
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
        if (STORE_AINV) {
            float* gai = a.ws.ainv + blk * C * C + r * C + j0;
            *reinterpret_cast<float4*>(gai) = x0;
            *reinterpret_cast<float4*>(gai + 4) = x1;
        }
        const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
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
                for (int e = 0; e < EV; ++e) f[e] = exp2f(sG[r * K + d0 + e]) * Vec16<T>::get(xk, e);
                *reinterpret_cast<uint4*>(sKg + r * LDK + d0) = Vec16<T>::pack(f);
            }
        }
        sKW = sKg;
        sAW = sA2;
    }
    __syncthreads();

    // ---- a4: W^T = K^T A1^T and U^T = V^T A2^T, tile (column block D of K or
    // V, token block I); the lane's 4 values are W[i][4 consecutive d]
    {
        T* gw = static_cast<T*>(a.ws.w) + blk * C * K;
        T* gu = static_cast<T*>(a.ws.u) + blk * C * V;
        constexpr int WJ = NB * (K / 16), UJ = NB * (V / 16);
        for (int job = wave; job < WJ + UJ; job += NW) {
            const bool isu = job >= WJ;
            const int jj = isu ? job - WJ : job;
            const int I = jj % NB, D = jj / NB;
            const int kn = min(C, ((16 * (I + 1) + KS - 1) / KS) * KS);
            const T* X = isu ? sV : sKW;              // [token][d]: k-major for X^T
            const int ldx = isu ? LDV : LDK;
            const T* Bt = (isu ? sA2 : sAW) + (16 * I + (lane & 15)) * LDC;
            f32x4 acc = zero4();
            for (int k0 = 0; k0 < kn; k0 += KS)
                acc = M::mma(M::load_t(X + k0 * ldx + 16 * D, ldx, lane), M::load(Bt + k0, lane),
                             acc);
            const int i = 16 * I + acc_col(lane);
            if (isu) store4(gu + i * V + 16 * D + 4 * (lane >> 4), acc);
            else store4(gw + i * K + 16 * D + 4 * (lane >> 4), acc);
        }
    }
}

template <typename T, int K, int V, int C, bool PK>
static hipError_t launch_intra_t(const IntraLaunch& a) {
    dim3 grid((unsigned)a.map.max_chunks, (unsigned)a.H);
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
