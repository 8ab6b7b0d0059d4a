// Inter-chunk state pass with the chunk output fused in (k4 + k5).
//
// The state h (K x V, fp32) is carried serially over the chunks of one
// (sequence, head); the value dimension is split into VT-wide tiles that run
// as independent workgroups.  Per chunk, with the intra-chunk products in the
// workspace (W, U, Qs = scale diag(gamma) Q, Ks = diag(gamma_C/gamma) K, Aqk):
//   V_new = U - W h                                    (MFMA)
//   O     = Qs h + Aqk V_new                           (MFMA)
//   h    <- gamma_C h + Ks^T V_new                     (MFMA, fp32 accumulate)
// ("TileLang 实战：KDA 从零到一--Gated DeltaNet" §2.3, eqs. 11-12, and §4.4
// order: the output reads the entering state, the state is decayed before the
// new contributions are added; "Gated Delta Network（GDN）" §4.1(d): the
// serial loop computes u - w h, decays h by the chunk-end gate and adds
// K^T V_new; "阅读笔记：DeltaNet 在 FLA 中的代码实现笔记", forward Steps 4-5.)
// For the per-key gate gamma_C is a vector and decays h row by row.
//
// Mapping (8 waves): each wave owns one (16-token, 16-value) tile of V_new
// and the matching transposed tile of O, and K/16 * VT/16 / 8 tiles of h,
// which stays in MFMA accumulators for the whole sequence.  A bf16 (or fp32)
// copy of h^T in LDS is the operand of the two products that read h, and
// V_new^T in LDS feeds the other two.  O is computed transposed so each
// lane stores 4 consecutive values of one output row straight to HBM.  The
// next chunk's operands are loaded into registers while the current chunk
// is computed and written to the other half of a double-buffered LDS area.
// The workgroups of one (sequence, head) get ids equal modulo 8, so the
// hardware's round-robin over the 8 XCDs puts them on one XCD and they share
// W, Qs, Ks and Aqk through its L2.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

constexpr int SCAN_THREADS = 512;

template <typename T, int K, int V, int C, int VT, bool PK>
struct ScanSmem {
    static constexpr int P = 16 / sizeof(T);
    static constexpr int LDK = K + P;     // [C][K] row-major: W, Qs, Ks; [VT][K] h^T
    static constexpr int LDC = C + P;     // [C][C] Aqk, [VT][C] V_new^T
    static constexpr int LDT = VT + P;    // [C][VT] U tile
    // one chunk's operands
    static constexpr size_t b_W = 0;
    static constexpr size_t b_Q = b_W + sizeof(T) * C * LDK;
    static constexpr size_t b_K = b_Q + sizeof(T) * C * LDK;
    static constexpr size_t b_A = b_K + sizeof(T) * C * LDK;
    static constexpr size_t b_U = b_A + sizeof(T) * C * LDC;
    static constexpr size_t b_D = b_U + sizeof(T) * C * LDT;
    static constexpr size_t BUF = ((b_D + sizeof(float) * (PK ? K : 4)) + 15) / 16 * 16;
    static constexpr size_t FIXED = sizeof(T) * VT * LDK + sizeof(T) * VT * LDC;
    static constexpr int NBUF = 2 * BUF + FIXED <= 160 * 1024 ? 2 : 1;
    static constexpr size_t o_hT = NBUF * BUF;
    static constexpr size_t o_Vn = o_hT + sizeof(T) * VT * LDK;
    static constexpr size_t bytes = o_Vn + sizeof(T) * VT * LDC;
};

// Registers holding the next chunk's operands between its load and its
// write to LDS.  The region of each slot is fixed at compile time (W, Qs, Ks
// are C*K/EV vectors each, Aqk C*C/EV, the U tile C*VT/EV; all multiples of
// 64, so partial passes are wave-uniform).
template <typename T, int PW, int PA, int PU>
struct ScanPrefetch {
    u32x4 w[PW], q[PW], k[PW], a[PA], u[PU];
    float d;

    template <int K, int V, int C, int VT, int NT, bool PK>
    __device__ __forceinline__ void issue(const T* gw, const T* gq, const T* gk, const T* ga,
                                          const T* gu, const float* gcum, int64_t blk, int v0,
                                          int tid) {
        constexpr int EV = 16 / sizeof(T);
        constexpr int NWV = C * K / EV, NAV = C * C / EV, NUV = C * VT / EV;
        const u32x4* w4 = reinterpret_cast<const u32x4*>(gw + blk * C * K);
        const u32x4* q4 = reinterpret_cast<const u32x4*>(gq + blk * C * K);
        const u32x4* k4 = reinterpret_cast<const u32x4*>(gk + blk * C * K);
        const u32x4* a4 = reinterpret_cast<const u32x4*>(ga + blk * C * C);
#pragma unroll
        for (int p = 0; p < PW; ++p) {
            const int i = tid + NT * p;
            if (NWV % NT == 0 || i < NWV) {
                w[p] = w4[i];
                q[p] = q4[i];
                k[p] = k4[i];
            }
        }
#pragma unroll
        for (int p = 0; p < PA; ++p) {
            const int i = tid + NT * p;
            if (NAV % NT == 0 || i < NAV) a[p] = a4[i];
        }
#pragma unroll
        for (int p = 0; p < PU; ++p) {
            const int i = tid + NT * p;
            if (NUV % NT == 0 || i < NUV) {
                const int r = i / (VT / EV), cv = i % (VT / EV);
                u[p] = *reinterpret_cast<const u32x4*>(gu + blk * C * V + r * V + v0 + cv * EV);
            }
        }
        if (PK) d = tid < K ? gcum[(blk * C + (C - 1)) * K + tid] : 0.f;
        else d = gcum[blk * C + (C - 1)];
    }

    template <typename L, int K, int C, int VT, int NT, bool PK>
    __device__ __forceinline__ void commit(char* buf, int tid) const {
        constexpr int EV = 16 / sizeof(T);
        constexpr int NWV = C * K / EV, NAV = C * C / EV, NUV = C * VT / EV;
        T* sW = reinterpret_cast<T*>(buf + L::b_W);
        T* sQ = reinterpret_cast<T*>(buf + L::b_Q);
        T* sK = reinterpret_cast<T*>(buf + L::b_K);
        T* sA = reinterpret_cast<T*>(buf + L::b_A);
        T* sU = reinterpret_cast<T*>(buf + L::b_U);
        float* sD = reinterpret_cast<float*>(buf + L::b_D);
#pragma unroll
        for (int p = 0; p < PW; ++p) {
            const int i = tid + NT * p;
            if (NWV % NT == 0 || i < NWV) {
                const int o = (i / (K / EV)) * L::LDK + (i % (K / EV)) * EV;
                *reinterpret_cast<u32x4*>(sW + o) = w[p];
                *reinterpret_cast<u32x4*>(sQ + o) = q[p];
                *reinterpret_cast<u32x4*>(sK + o) = k[p];
            }
        }
#pragma unroll
        for (int p = 0; p < PA; ++p) {
            const int i = tid + NT * p;
            if (NAV % NT == 0 || i < NAV)
                *reinterpret_cast<u32x4*>(sA + (i / (C / EV)) * L::LDC + (i % (C / EV)) * EV) = a[p];
        }
#pragma unroll
        for (int p = 0; p < PU; ++p) {
            const int i = tid + NT * p;
            if (NUV % NT == 0 || i < NUV)
                *reinterpret_cast<u32x4*>(sU + (i / (VT / EV)) * L::LDT + (i % (VT / EV)) * EV) = u[p];
        }
        if (PK) {
            if (tid < K) sD[tid] = exp2f(d);
        } else if (tid == 0) {
            sD[0] = exp2f(d);
        }
    }
};

template <typename T, int K, int V, int C, int VT, bool PK>
__global__ __launch_bounds__(SCAN_THREADS) void scan_kernel(ScanLaunch a) {
    typedef ScanSmem<T, K, V, C, VT, PK> L;
    typedef Mma<T> M;
    constexpr int NT = SCAN_THREADS, NW = NT / 64;
    constexpr int LDK = L::LDK, LDC = L::LDC, LDT = L::LDT;
    constexpr int KS = M::KSTEP;
    constexpr int EV = 16 / sizeof(T);
    constexpr int NVT = V / VT;
    constexpr int CT = VT / 16;              // value tiles
    constexpr int TT = C / 16;               // token tiles
    constexpr int NHT = (K / 16) * CT;       // h tiles
    constexpr int HPW = (NHT + NW - 1) / NW; // h tiles per wave
    static_assert(TT * CT <= NW, "one V_new tile per wave");
    static_assert(K % 16 == 0 && VT % 16 == 0 && V % VT == 0, "tile shape");
    __shared__ __attribute__((aligned(16))) char smem[L::bytes];
    T* shT = reinterpret_cast<T*>(smem + L::o_hT);
    T* sVn = reinterpret_cast<T*>(smem + L::o_Vn);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t bid = blockIdx.x;
    const int vt = (int)((bid >> 3) % NVT);
    const int64_t chain = (bid & 7) + 8 * ((bid >> 3) / NVT);
    if (chain >= a.N * a.H) return;
    const int64_t n = chain / a.H, h = chain - n * a.H;
    const int v0 = vt * VT;

    int64_t t0, len, c0;
    if (a.map.seqs) {
        const int4 s = a.map.seqs[n];
        t0 = s.x;
        len = s.y;
        c0 = s.z;
    } else {
        t0 = n * a.map.T;
        len = a.map.T;
        c0 = n * a.map.nt;
    }

    // ---- h tiles owned by this wave: tile id = wave + NW * s -> (row block, value tile)
    f32x4 hacc[HPW];
    const float* h0 = a.h0 ? a.h0 + (n * a.H + h) * (int64_t)(K * V) : nullptr;
#pragma unroll
    for (int s = 0; s < HPW; ++s) {
        const int id = wave + NW * s;
        hacc[s] = zero4();
        if (id < NHT) {
            const int rb = 16 * (id / CT), ct = id % CT;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                hacc[s][e] = h0 ? h0[(rb + acc_row(lane, e)) * V + v0 + 16 * ct + acc_col(lane)]
                                : 0.f;
            store_acc_t(shT + (16 * ct) * LDK + rb, LDK, lane, hacc[s]);
        }
    }

    // ---- chunk operands, 16-byte vectors; the region of each register slot is
    // fixed at compile time (W, Qs, Ks are C*K/EV vectors each, Aqk C*C/EV,
    // the U tile C*VT/EV; all multiples of 64, so partial passes are
    // wave-uniform)
    constexpr int NWV = C * K / EV, NAV = C * C / EV, NUV = C * VT / EV;
    constexpr int PW = (NWV + NT - 1) / NT, PA = (NAV + NT - 1) / NT, PU = (NUV + NT - 1) / NT;
    static_assert(NWV % 64 == 0 && NAV % 64 == 0 && NUV % 64 == 0, "wave-uniform passes");
    ScanPrefetch<T, PW, PA, PU> pre;
    const T* gw = static_cast<const T*>(a.ws.w);
    const T* gq = static_cast<const T*>(a.ws.qs);
    const T* gk = static_cast<const T*>(a.ws.ks);
    const T* ga = static_cast<const T*>(a.ws.aqk);
    const T* gu = static_cast<const T*>(a.ws.u);
#define GDN_SCAN_ISSUE(BLK)                                                                   \
    pre.template issue<K, V, C, VT, NT, PK>(gw, gq, gk, ga, gu, a.ws.gcum, (BLK), v0, tid)
#define GDN_SCAN_COMMIT(BUF)                                                                  \
    pre.template commit<L, K, C, VT, NT, PK>((BUF), tid)

    const int nch = (int)((len + C - 1) / C);
    T* o = static_cast<T*>(a.o);
    // this wave's V_new / O tile
    const int tt = wave % TT, ct = wave / TT;
    const bool has_tile = wave < TT * CT;
    if (nch > 0 && c0 < a.map.max_chunks) {
        GDN_SCAN_ISSUE(h * a.map.max_chunks + c0);
        GDN_SCAN_COMMIT(smem);
    }
    __syncthreads();
    for (int j = 0; j < nch; ++j) {
        const int64_t c = c0 + j;
        if (c >= a.map.max_chunks) break;
        char* buf = smem + (L::NBUF == 2 ? (j & 1) * L::BUF : 0);
        const T* sW = reinterpret_cast<const T*>(buf + L::b_W);
        const T* sQ = reinterpret_cast<const T*>(buf + L::b_Q);
        const T* sK = reinterpret_cast<const T*>(buf + L::b_K);
        const T* sA = reinterpret_cast<const T*>(buf + L::b_A);
        const T* sU = reinterpret_cast<const T*>(buf + L::b_U);
        const float* sD = reinterpret_cast<const float*>(buf + L::b_D);
        const int64_t tt0 = t0 + (int64_t)j * C;
        const int ntok = (int)min((int64_t)C, len - (int64_t)j * C);
        const bool more = j + 1 < nch && c + 1 < a.map.max_chunks;
        if (more) GDN_SCAN_ISSUE(h * a.map.max_chunks + c + 1);

        // ---- V_new = U - W h (tile tokens tt x values ct) and
        //      O^T = h^T Qs^T (tile values ct x tokens tt); both read the same
        //      h^T fragment (as B in the first product, as A in the second)
        f32x4 ov = zero4();
        if (has_tile) {
            f32x4 vn = zero4();
            const T* wr = sW + (16 * tt + (lane & 15)) * LDK;
            const T* qr = sQ + (16 * tt + (lane & 15)) * LDK;
            const T* hr = shT + (16 * ct + (lane & 15)) * LDK;
            float u[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                u[e] = Elem<T>::load(sU + (16 * tt + acc_row(lane, e)) * LDT + 16 * ct +
                                     acc_col(lane));
#pragma unroll
            for (int k0 = 0; k0 < K; k0 += KS) {
                const typename M::frag fh = M::load(hr + k0, lane);
                vn = M::mma(M::load(wr + k0, lane), fh, vn);
                ov = M::mma(fh, M::load(qr + k0, lane), ov);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) vn[e] = u[e] - vn[e];
            store_acc_t(sVn + (16 * ct) * LDC + 16 * tt, LDC, lane, vn);   // V_new^T
        }
        __syncthreads();

        // ---- O^T += V_new^T Aqk^T, store O; h <- gamma_C h + Ks^T V_new
        if (has_tile) {
            const int kn = min(C, ((16 * (tt + 1) + KS - 1) / KS) * KS);
            ov = mma_tile<T>(sVn + 16 * ct * LDC, LDC, sA + 16 * tt * LDC, LDC, kn, lane, ov);
            const int tok = 16 * tt + acc_col(lane);
            if (tok < ntok)
                store4(o + ((tt0 + tok) * a.H + h) * V + v0 + 16 * ct + 4 * (lane >> 4), ov);
        }
#pragma unroll
        for (int s = 0; s < HPW; ++s) {
            const int id = wave + NW * s;
            if (id < NHT) {
                const int rb = 16 * (id / CT), hc = id % CT;
#pragma unroll
                for (int e = 0; e < 4; ++e) hacc[s][e] *= PK ? sD[rb + acc_row(lane, e)] : sD[0];
                const T* vr = sVn + (16 * hc + (lane & 15)) * LDC;
#pragma unroll
                for (int k0 = 0; k0 < C; k0 += KS)
                    hacc[s] = M::mma(M::load_t(sK + k0 * LDK + rb, LDK, lane), M::load(vr + k0, lane),
                                     hacc[s]);
                store_acc_t(shT + (16 * hc) * LDK + rb, LDK, lane, hacc[s]);
            }
        }
        if (more) {
            if (L::NBUF == 2) {
                GDN_SCAN_COMMIT(smem + ((j + 1) & 1) * L::BUF);
            } else {
                __syncthreads();   // single buffer: every wave is done with this chunk
                GDN_SCAN_COMMIT(smem);
            }
        }
        __syncthreads();
    }

#undef GDN_SCAN_ISSUE
#undef GDN_SCAN_COMMIT
    if (a.ht) {
        float* ht = a.ht + (n * a.H + h) * (int64_t)(K * V);
#pragma unroll
        for (int s = 0; s < HPW; ++s) {
            const int id = wave + NW * s;
            if (id < NHT) {
                const int rb = 16 * (id / CT), hc = id % CT;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    ht[(rb + acc_row(lane, e)) * V + v0 + 16 * hc + acc_col(lane)] = hacc[s][e];
            }
        }
    }
}

template <typename T, int K, int V, int C, int VT, bool PK>
static hipError_t launch_scan_t(const ScanLaunch& a) {
    const int64_t chains = a.N * a.H;
    const int64_t nblk = ((chains + 7) / 8) * 8 * (V / VT);
    hipLaunchKernelGGL((scan_kernel<T, K, V, C, VT, PK>), dim3((unsigned)nblk), dim3(SCAN_THREADS),
                       0, a.stream, a);
    return hipGetLastError();
}

template <typename T, int VT>
static hipError_t launch_scan_dt(const ScanLaunch& a) {
#define GDN_SCAN_CASE(KK, VV)                                                    \
    if (a.K == KK && a.V == VV)                                                  \
        return a.per_key ? launch_scan_t<T, KK, VV, 64, VT, true>(a)             \
                         : launch_scan_t<T, KK, VV, 64, VT, false>(a);
    GDN_SCAN_CASE(64, 64)
    GDN_SCAN_CASE(64, 128)
    GDN_SCAN_CASE(128, 64)
    GDN_SCAN_CASE(128, 128)
#undef GDN_SCAN_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_scan(const ScanLaunch& a) {
    if (a.C != 64) return hipErrorInvalidValue;
    return a.bf16 ? launch_scan_dt<bf16, 32>(a) : launch_scan_dt<float, 32>(a);
}

}  // namespace gdn
