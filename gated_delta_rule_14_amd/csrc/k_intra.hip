// Intra-chunk stage: everything about a chunk that does not depend on the
// state entering it.  One 256-thread workgroup per (chunk, head); all chunks
// of all heads run in parallel.
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
// and, for the state pass, Qs = scale Q diag(gamma) and Kt = (K gamma_C/gamma)^T.
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
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

template <typename T, int K, int V, int C, bool PK>
struct IntraSmem {
    static constexpr int P = 16 / sizeof(T);  // 16-byte row padding
    static constexpr int LDK = K + P;         // row-major [C][K]
    static constexpr int LDV = V + P;         // row-major [C][V]
    static constexpr int LDC = C + P;         // n-major [K or V][C]
    static constexpr int LDA = C + 1;         // fp32 [C][C]
    static constexpr int NB = C / 16;
    static constexpr int SCR_ROWS = 2 * 16 + C - 16;   // per-key scaled operands
    // A (fp32, for the solve) and then (beta V)^T share one region
    static constexpr size_t AV_BYTES = sizeof(float) * C * LDA > sizeof(T) * V * LDC
                                           ? sizeof(float) * C * LDA : sizeof(T) * V * LDC;
    static constexpr size_t o_K = 0;
    static constexpr size_t o_Q = o_K + sizeof(T) * C * LDK;
    static constexpr size_t o_KT = o_Q + sizeof(T) * C * LDK;
    static constexpr size_t o_AV = o_KT + sizeof(T) * K * LDC;
    static constexpr size_t o_G = o_AV + ((AV_BYTES + 15) / 16) * 16;
    static constexpr size_t o_B = o_G + sizeof(float) * C * (PK ? K : 1);
    static constexpr size_t o_P = o_B + sizeof(float) * C;
    static constexpr size_t o_S = o_P + sizeof(float) * 4 * 16 * 17;
    static constexpr size_t bytes = o_S + (PK ? sizeof(T) * SCR_ROWS * LDK : 0);
    static_assert(C * LDC <= K * LDC, "Aqk staging must fit the K^T buffer");
    static_assert(sizeof(T) * C * LDV <= AV_BYTES, "U staging must fit the A / V^T region");
    static_assert(C * LDC <= C * LDK, "Ainv copy must fit the Q buffer");
};

template <typename T, int K, int V, int C, bool PK, bool STORE_AINV>
__global__ __launch_bounds__(256) void intra_kernel(IntraLaunch a) {
    typedef IntraSmem<T, K, V, C, PK> L;
    constexpr int LDK = L::LDK, LDV = L::LDV, LDC = L::LDC, LDA = L::LDA, NB = L::NB;
    constexpr int EV = 16 / sizeof(T);
    constexpr int KS = Mma<T>::KSTEP;
    __shared__ __attribute__((aligned(16))) char smem[L::bytes];
    T* sK = reinterpret_cast<T*>(smem + L::o_K);
    T* sQ = reinterpret_cast<T*>(smem + L::o_Q);
    T* sKT = reinterpret_cast<T*>(smem + L::o_KT);
    float* sA = reinterpret_cast<float*>(smem + L::o_AV);   // until Ainv is copied out
    T* sVT = reinterpret_cast<T*>(smem + L::o_AV);          // after that
    float* sG = reinterpret_cast<float*>(smem + L::o_G);
    float* sB = reinterpret_cast<float*>(smem + L::o_B);
    float* sP = reinterpret_cast<float*>(smem + L::o_P);
    T* sStage = sKT;     // Aqk staging (before K^T is built)
    T* sAb = sQ;         // Ainv in the element type (after Q is consumed)

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
            if (r < C) {
                sG[r] = G;
                sB[r] = bt;
            }
        }
    } else {
        for (int d = tid; d < K; d += 256) {
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
        for (int r = tid; r < C; r += 256) sB[r] = r < n ? a.beta[(t0 + r) * H + h] : 0.f;
    }
    // K, Q, V rows: every load issued before any is used (zeros past n)
    constexpr int VK = C * (K / EV), VV = C * (V / EV);
    constexpr int PK_ = (VK + 255) / 256, PV = (VV + 255) / 256;
    uint4 kreg[PK_], qreg[PK_], vreg[PV];
#pragma unroll
    for (int p = 0; p < PK_; ++p) {
        const int i = tid + 256 * p, r = i / (K / EV), cv = i - r * (K / EV);
        kreg[p] = qreg[p] = make_uint4(0, 0, 0, 0);
        if (i < VK && r < n) {
            kreg[p] = *reinterpret_cast<const uint4*>(k + ((t0 + r) * H + h) * K + cv * EV);
            qreg[p] = *reinterpret_cast<const uint4*>(q + ((t0 + r) * H + h) * K + cv * EV);
        }
    }
#pragma unroll
    for (int p = 0; p < PV; ++p) {
        const int i = tid + 256 * p, r = i / (V / EV), cv = i - r * (V / EV);
        vreg[p] = make_uint4(0, 0, 0, 0);
        if (i < VV && r < n)
            vreg[p] = *reinterpret_cast<const uint4*>(v + ((t0 + r) * H + h) * V + cv * EV);
    }
#pragma unroll
    for (int p = 0; p < PK_; ++p) {
        const int i = tid + 256 * p, r = i / (K / EV), cv = i - r * (K / EV);
        if (i < VK) {
            *reinterpret_cast<uint4*>(sK + r * LDK + cv * EV) = kreg[p];
            *reinterpret_cast<uint4*>(sQ + r * LDK + cv * EV) = qreg[p];
        }
    }
    // zero A and the Aqk staging area
    for (int i = tid; i < C * C; i += 256) {
        const int r = i / C, j = i - r * C;
        sA[r * LDA + j] = 0.f;
        Elem<T>::store(sStage + r * LDC + j, 0.f);
    }
    __syncthreads();

    // ---- a2: beta-scaled decay-masked strictly-lower K K^T and causal Q K^T
    if (!PK) {
        constexpr int NT2 = NB * (NB + 1) / 2;
        for (int job = wave; job < 2 * NT2; job += 4) {
            const bool isq = job >= NT2;
            int t = isq ? job - NT2 : job, I = 0;
            while (t > I) { t -= I + 1; ++I; }
            const int J = t;
            const T* A0 = (isq ? sQ : sK) + 16 * I * LDK;
            f32x4 acc = mma_tile<T>(A0, LDK, sK + 16 * J * LDK, LDK, K, lane, zero4());
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * I + acc_row(lane, e), j = 16 * J + acc_col(lane);
                const float dec = exp2f(fminf(sG[i] - sG[j], 0.f));
                if (!isq) {
                    if (j < i) sA[i * LDA + j] = sB[i] * dec * acc[e];
                } else if (j <= i) {
                    Elem<T>::store(sStage + i * LDC + j, a.scale * dec * acc[e]);
                }
            }
        }
    } else {
        T* sS = reinterpret_cast<T*>(smem + L::o_S);
        for (int I = 1; I < NB; ++I) {
            const int b = 16 * I;
            __syncthreads();   // previous I's tiles have read the scratch
            // rows [0,16): K_I 2^{G_I - G_b}; [16,32): Q_I 2^{G_I - G_b};
            // [32, 32 + b): K_J 2^{G_b - G_J} for all J < I
            for (int i = tid; i < (32 + b) * K; i += 256) {
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
            for (int job = wave; job < 2 * I; job += 4) {
                const bool isq = job >= I;
                const int J = isq ? job - I : job;
                f32x4 acc = mma_tile<T>(sS + (isq ? 16 : 0) * LDK, LDK, sS + (32 + 16 * J) * LDK,
                                        LDK, K, lane, zero4());
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 16 * I + acc_row(lane, e), j = 16 * J + acc_col(lane);
                    if (!isq) sA[i * LDA + j] = sB[i] * acc[e];
                    else Elem<T>::store(sStage + i * LDC + j, a.scale * acc[e]);
                }
            }
        }
        // diagonal 16x16 blocks, pair by pair: thread = (block, row, quarter of d)
        {
            constexpr int DQ = K / 4;
            const int I = tid >> 6, i = 16 * I + ((tid & 63) >> 2), s = tid & 3;
            if (I < NB) {
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
                    akk += __shfl_xor(akk, 1, 64);
                    akk += __shfl_xor(akk, 2, 64);
                    aqk += __shfl_xor(aqk, 1, 64);
                    aqk += __shfl_xor(aqk, 2, 64);
                    if (s == 0 && j <= i) {
                        if (j < i) sA[i * LDA + j] = sB[i] * akk;
                        Elem<T>::store(sStage + i * LDC + j, a.scale * aqk);
                    }
                }
            }
        }
    }
    __syncthreads();

    // ---- outputs that need only G, Q, K: Aqk, Qs, Kt, gcum
    {
        T* gaqk = static_cast<T*>(a.ws.aqk) + blk * C * C;
        copy_tile<T>(gaqk, C, sStage, LDC, C, C, tid, 256);
        T* gqs = static_cast<T*>(a.ws.qs) + blk * C * K;
        for (int i = tid; i < C * (K / EV); i += 256) {
            const int r = i / (K / EV), d0 = (i - r * (K / EV)) * EV;
            const uint4 x = *reinterpret_cast<const uint4*>(sQ + r * LDK + d0);
            float f[EV];
#pragma unroll
            for (int e = 0; e < EV; ++e)
                f[e] = a.scale * exp2f(PK ? sG[r * K + d0 + e] : sG[r]) * Vec16<T>::get(x, e);
            *reinterpret_cast<uint4*>(gqs + r * K + d0) = Vec16<T>::pack(f);
        }
        // Kt[d][r] = k[r][d] * 2^{G_C-1 - G_r}: 8 tokens per 16-byte store (bf16)
        T* gkt = static_cast<T*>(a.ws.kt) + blk * K * C;
        for (int i = tid; i < K * (C / EV); i += 256) {
            const int d = i / (C / EV), r0 = (i - d * (C / EV)) * EV;
            float f[EV];
#pragma unroll
            for (int e = 0; e < EV; ++e) {
                const int r = r0 + e;
                const float gl = PK ? sG[(C - 1) * K + d] - sG[r * K + d] : sG[C - 1] - sG[r];
                f[e] = Elem<T>::load(sK + r * LDK + d) * exp2f(fminf(gl, 0.f));
            }
            *reinterpret_cast<uint4*>(gkt + d * C + r0) = Vec16<T>::pack(f);
        }
        float* gg = a.ws.gcum + blk * C * (PK ? K : 1);
        for (int i = tid; i < C * (PK ? K : 1); i += 256) gg[i] = sG[i];
    }
    __syncthreads();

    // ---- (beta gamma K)^T into sKT: the B operand of W
    for (int i = tid; i < K * (C / EV); i += 256) {
        const int d = i / (C / EV), r0 = (i - d * (C / EV)) * EV;
        float f[EV];
#pragma unroll
        for (int e = 0; e < EV; ++e) {
            const int r = r0 + e;
            const float gm = exp2f(PK ? sG[r * K + d] : sG[r]);
            f[e] = sB[r] * gm * Elem<T>::load(sK + r * LDK + d);
        }
        *reinterpret_cast<uint4*>(sKT + d * LDC + r0) = Vec16<T>::pack(f);
    }

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
    if (STORE_AINV) {
        float* gai = a.ws.ainv + blk * C * C;
        for (int i = tid; i < C * C; i += 256) gai[i] = sA[(i / C) * LDA + (i % C)];
    }
    // Ainv in the element type, row-major [C][LDC]
    for (int i = tid; i < C * C; i += 256) {
        const int r = i / C, j = i - r * C;
        Elem<T>::store(sAb + r * LDC + j, sA[r * LDA + j]);
    }
    __syncthreads();
    // (beta V)^T, the B operand of U, into the region A occupied
#pragma unroll
    for (int p = 0; p < PV; ++p) {
        const int i = tid + 256 * p, r = i / (V / EV), cv = i - r * (V / EV);
        if (i < VV) {
            const float bt = sB[r];
#pragma unroll
            for (int e = 0; e < EV; ++e)
                Elem<T>::store(sVT + (cv * EV + e) * LDC + r, bt * Vec16<T>::get(vreg[p], e));
        }
    }
    __syncthreads();

    // ---- a4: W = Ainv (beta gamma K), U = Ainv (beta V)
    constexpr int WJ = NB * (K / 16), UJ = NB * (V / 16);
    constexpr int WPW = (WJ + 3) / 4, UPW = (UJ + 3) / 4;
    f32x4 wacc[WPW], uacc[UPW];
#pragma unroll
    for (int s = 0; s < WPW; ++s) {
        const int job = wave + 4 * s;
        wacc[s] = zero4();
        if (job < WJ) {
            const int I = job % NB, D = job / NB;
            const int kn = min(C, ((16 * (I + 1) + KS - 1) / KS) * KS);
            wacc[s] = mma_tile<T>(sAb + 16 * I * LDC, LDC, sKT + 16 * D * LDC, LDC, kn, lane,
                                  zero4());
        }
    }
#pragma unroll
    for (int s = 0; s < UPW; ++s) {
        const int job = wave + 4 * s;
        uacc[s] = zero4();
        if (job < UJ) {
            const int I = job % NB, D = job / NB;
            const int kn = min(C, ((16 * (I + 1) + KS - 1) / KS) * KS);
            uacc[s] = mma_tile<T>(sAb + 16 * I * LDC, LDC, sVT + 16 * D * LDC, LDC, kn, lane,
                                  zero4());
        }
    }
    __syncthreads();
    T* sWst = sK;    // [C][LDK]
    T* sUst = sVT;   // [C][LDV]
#pragma unroll
    for (int s = 0; s < WPW; ++s) {
        const int job = wave + 4 * s;
        if (job < WJ) {
            const int I = job % NB, D = job / NB;
            store_acc<T>(sWst + 16 * I * LDK + 16 * D, LDK, lane, wacc[s]);
        }
    }
#pragma unroll
    for (int s = 0; s < UPW; ++s) {
        const int job = wave + 4 * s;
        if (job < UJ) {
            const int I = job % NB, D = job / NB;
            store_acc<T>(sUst + 16 * I * LDV + 16 * D, LDV, lane, uacc[s]);
        }
    }
    __syncthreads();
    copy_tile<T>(static_cast<T*>(a.ws.w) + blk * C * K, K, sWst, LDK, C, K, tid, 256);
    copy_tile<T>(static_cast<T*>(a.ws.u) + blk * C * V, V, sUst, LDV, C, V, tid, 256);
}

template <typename T, int K, int V, int C, bool PK>
static hipError_t launch_intra_t(const IntraLaunch& a) {
    dim3 grid((unsigned)a.map.max_chunks, (unsigned)a.H);
    if (a.ws.ainv)
        hipLaunchKernelGGL((intra_kernel<T, K, V, C, PK, true>), grid, dim3(256), 0, a.stream, a);
    else
        hipLaunchKernelGGL((intra_kernel<T, K, V, C, PK, false>), grid, dim3(256), 0, a.stream, a);
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
