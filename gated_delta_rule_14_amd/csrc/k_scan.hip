// Inter-chunk state pass with the chunk output fused in (k4 + k5).
//
// The state h (K x V, fp32) is carried serially over the chunks of one
// (sequence, head); the value dimension is split into VT-wide tiles that run
// as independent workgroups.  Per chunk, with the intra-chunk products in the
// workspace (W, U, Qs = scale Q diag(gamma), Kt = (K gamma_C/gamma)^T, Aqk):
//   V_new = U - W h                                    (MFMA)
//   O     = Qs h + Aqk V_new                           (MFMA)
//   h    <- gamma_C h + Kt V_new                       (MFMA, fp32 accumulate)
// ("TileLang 实战：KDA 从零到一--Gated DeltaNet" §2.3, eqs. 11-12, and §4.4
// order: the output reads the entering state, the state is decayed before the
// new contributions are added; "Gated Delta Network（GDN）" §4.1(d): the
// serial loop computes u - w h, decays h by the chunk-end gate and adds
// K^T V_new; "阅读笔记：DeltaNet 在 FLA 中的代码实现笔记", forward Steps 4-5.)
// For the per-key gate gamma_C is a vector and decays h row by row.
//
// h stays in MFMA accumulators for the whole sequence; a bf16 (or fp32)
// copy of h^T in LDS is the B operand of the two products that read it.
// Workgroups of one (sequence, head) are placed on the same XCD (the hardware
// deals workgroups round-robin over the 8 XCDs), so they share W, Qs, Kt and
// Aqk through that XCD's L2.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

template <typename T, int K, int V, int C, int VT>
struct ScanSmem {
    static constexpr int P = 16 / sizeof(T);
    static constexpr int LDK = K + P;     // [C][K] row-major, [VT][K] h^T
    static constexpr int LDC = C + P;     // [K][C] Kt, [C][C] Aqk, [VT][C] V_new^T
    static constexpr int LDT = VT + P;    // [C][VT] U tile and O tile
    static constexpr size_t o_W = 0;
    static constexpr size_t o_Q = o_W + sizeof(T) * C * LDK;
    static constexpr size_t o_Kt = o_Q + sizeof(T) * C * LDK;
    static constexpr size_t o_Aqk = o_Kt + sizeof(T) * K * LDC;
    static constexpr size_t o_U = o_Aqk + sizeof(T) * C * LDC;
    static constexpr size_t o_O = o_U + sizeof(T) * C * LDT;
    static constexpr size_t o_hT = o_O + sizeof(T) * C * LDT;
    static constexpr size_t o_Vn = o_hT + sizeof(T) * VT * LDK;
    static constexpr size_t o_D = o_Vn + sizeof(T) * VT * LDC;
    static constexpr size_t bytes = o_D + sizeof(float) * K;
};

template <typename T, int K, int V, int C, int VT, bool PK>
__global__ __launch_bounds__(256) void scan_kernel(ScanLaunch a) {
    typedef ScanSmem<T, K, V, C, VT> L;
    constexpr int LDK = L::LDK, LDC = L::LDC, LDT = L::LDT;
    constexpr int KS = Mma<T>::KSTEP;
    constexpr int NVT = V / VT;
    constexpr int RT = K / 64;      // 16-row h tiles per wave
    constexpr int CT = VT / 16;     // 16-col tiles
    static_assert(K % 64 == 0 && VT % 16 == 0 && V % VT == 0, "tile shape");
    __shared__ __attribute__((aligned(16))) char smem[L::bytes];
    T* sW = reinterpret_cast<T*>(smem + L::o_W);
    T* sQ = reinterpret_cast<T*>(smem + L::o_Q);
    T* sKt = reinterpret_cast<T*>(smem + L::o_Kt);
    T* sAqk = reinterpret_cast<T*>(smem + L::o_Aqk);
    T* sU = reinterpret_cast<T*>(smem + L::o_U);
    T* sO = reinterpret_cast<T*>(smem + L::o_O);
    T* shT = reinterpret_cast<T*>(smem + L::o_hT);
    T* sVn = reinterpret_cast<T*>(smem + L::o_Vn);
    float* sD = reinterpret_cast<float*>(smem + L::o_D);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // XCD-aware placement: the NVT tiles of a chain get ids that are equal
    // modulo 8, i.e. land on the same XCD.
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

    // h: wave w owns rows [w*K/4, (w+1)*K/4), all VT columns
    f32x4 hacc[RT][CT];
    const float* h0 = a.h0 ? a.h0 + (n * a.H + h) * (int64_t)(K * V) : nullptr;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = wave * (K / 4) + 16 * rt + acc_row(lane, e);
                const int col = v0 + 16 * ct + acc_col(lane);
                hacc[rt][ct][e] = h0 ? h0[row * V + col] : 0.f;
            }
            store_acc_t(shT + (16 * ct) * LDK + wave * (K / 4) + 16 * rt, LDK, lane,
                        hacc[rt][ct]);
        }

    // ---- chunk operands: W, Qs [C][K], Kt [K][C], Aqk [C][C], U tile [C][VT],
    // moved as 16-byte vectors.  Chunk j+1 is loaded into registers while
    // chunk j is computed, then written to LDS.
    constexpr int EV = 16 / sizeof(T);
    constexpr int VW = C * K / EV, VQ = C * K / EV, VK = K * C / EV, VA = C * C / EV,
                  VU = C * VT / EV;
    constexpr int NV = VW + VQ + VK + VA + VU;
    constexpr int PER = (NV + 255) / 256;
    uint4 pre[PER];
    float pre_d = 0.f;
    const T* gw = static_cast<const T*>(a.ws.w);
    const T* gq = static_cast<const T*>(a.ws.qs);
    const T* gk = static_cast<const T*>(a.ws.kt);
    const T* ga = static_cast<const T*>(a.ws.aqk);
    const T* gu = static_cast<const T*>(a.ws.u);
    auto issue = [&](int64_t blk) {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int i = tid + 256 * p;
            const uint4* src;
            if (i < VW) src = reinterpret_cast<const uint4*>(gw + blk * C * K) + i;
            else if (i < VW + VQ) src = reinterpret_cast<const uint4*>(gq + blk * C * K) + (i - VW);
            else if (i < VW + VQ + VK)
                src = reinterpret_cast<const uint4*>(gk + blk * K * C) + (i - VW - VQ);
            else if (i < VW + VQ + VK + VA)
                src = reinterpret_cast<const uint4*>(ga + blk * C * C) + (i - VW - VQ - VK);
            else if (i < NV) {
                const int u = i - (VW + VQ + VK + VA), r = u / (VT / EV), cv = u - r * (VT / EV);
                src = reinterpret_cast<const uint4*>(gu + blk * C * V + r * V + v0) + cv;
            } else {
                src = nullptr;
            }
            pre[p] = src ? *src : make_uint4(0, 0, 0, 0);
        }
        if (PK) pre_d = tid < K ? a.ws.gcum[(blk * C + (C - 1)) * K + tid] : 0.f;
        else pre_d = a.ws.gcum[blk * C + (C - 1)];
    };
    float dsc = 0.f;
    auto commit = [&]() {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int i = tid + 256 * p;
            T* dst;
            if (i < VW) {
                const int r = i / (K / EV), cv = i - r * (K / EV);
                dst = sW + r * LDK + cv * EV;
            } else if (i < VW + VQ) {
                const int u = i - VW, r = u / (K / EV), cv = u - r * (K / EV);
                dst = sQ + r * LDK + cv * EV;
            } else if (i < VW + VQ + VK) {
                const int u = i - VW - VQ, r = u / (C / EV), cv = u - r * (C / EV);
                dst = sKt + r * LDC + cv * EV;
            } else if (i < VW + VQ + VK + VA) {
                const int u = i - VW - VQ - VK, r = u / (C / EV), cv = u - r * (C / EV);
                dst = sAqk + r * LDC + cv * EV;
            } else if (i < NV) {
                const int u = i - (VW + VQ + VK + VA), r = u / (VT / EV), cv = u - r * (VT / EV);
                dst = sU + r * LDT + cv * EV;
            } else {
                dst = nullptr;
            }
            if (dst) *reinterpret_cast<uint4*>(dst) = pre[p];
        }
        if (PK) {
            if (tid < K) sD[tid] = exp2f(pre_d);
        } else {
            dsc = exp2f(pre_d);
        }
    };

    const int nch = (int)((len + C - 1) / C);
    T* o = static_cast<T*>(a.o);
    if (nch > 0 && c0 < a.map.max_chunks) {
        issue(h * a.map.max_chunks + c0);
        commit();
    }
    __syncthreads();
    for (int j = 0; j < nch; ++j) {
        const int64_t c = c0 + j;
        if (c >= a.map.max_chunks) break;
        const int64_t tt0 = t0 + (int64_t)j * C;
        const int ntok = (int)min((int64_t)C, len - (int64_t)j * C);
        const bool more = j + 1 < nch && c + 1 < a.map.max_chunks;
        if (more) issue(h * a.map.max_chunks + c + 1);
        const float dcur = dsc;

        // ---- V_new = U - W h and O = Qs h, one 16-row tile per wave
        f32x4 ov[CT];
        if (wave < C / 16) {
            f32x4 vn[CT];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                vn[ct] = zero4();
                ov[ct] = zero4();
            }
            const T* wr = sW + (16 * wave + (lane & 15)) * LDK;
            const T* qr = sQ + (16 * wave + (lane & 15)) * LDK;
#pragma unroll
            for (int k0 = 0; k0 < K; k0 += KS) {
                const typename Mma<T>::frag fw = Mma<T>::load(wr + k0, lane);
                const typename Mma<T>::frag fq = Mma<T>::load(qr + k0, lane);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const typename Mma<T>::frag fh =
                        Mma<T>::load(shT + (16 * ct + (lane & 15)) * LDK + k0, lane);
                    vn[ct] = Mma<T>::mma(fw, fh, vn[ct]);
                    ov[ct] = Mma<T>::mma(fq, fh, ov[ct]);
                }
            }
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * wave + acc_row(lane, e);
                    vn[ct][e] = Elem<T>::load(sU + r * LDT + 16 * ct + acc_col(lane)) - vn[ct][e];
                }
                store_acc_t(sVn + (16 * ct) * LDC + 16 * wave, LDC, lane, vn[ct]);
            }
        }
        __syncthreads();

        // ---- O += Aqk V_new; h <- gamma_C h + Kt V_new
        if (wave < C / 16) {
            const int kn = min(C, ((16 * (wave + 1) + KS - 1) / KS) * KS);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                ov[ct] = mma_tile<T>(sAqk + 16 * wave * LDC, LDC, sVn + 16 * ct * LDC, LDC, kn,
                                     lane, ov[ct]);
                store_acc<T>(sO + 16 * wave * LDT + 16 * ct, LDT, lane, ov[ct]);
            }
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int rb = wave * (K / 4) + 16 * rt;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    hacc[rt][ct][e] *= PK ? sD[rb + acc_row(lane, e)] : dcur;
                hacc[rt][ct] = mma_tile<T>(sKt + rb * LDC, LDC, sVn + 16 * ct * LDC, LDC, C, lane,
                                           hacc[rt][ct]);
                store_acc_t(shT + (16 * ct) * LDK + rb, LDK, lane, hacc[rt][ct]);
            }
        }
        __syncthreads();

        // ---- O tile to HBM (rows past the end of the sequence are dropped),
        // then the prefetched chunk into LDS
        for (int i = tid; i < ntok * (VT / EV); i += 256) {
            const int r = i / (VT / EV), cv = i - r * (VT / EV);
            *reinterpret_cast<uint4*>(o + ((tt0 + r) * a.H + h) * V + v0 + cv * EV) =
                *reinterpret_cast<const uint4*>(sO + r * LDT + cv * EV);
        }
        if (more) commit();
        __syncthreads();
    }

    if (a.ht) {
        float* ht = a.ht + (n * a.H + h) * (int64_t)(K * V);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = wave * (K / 4) + 16 * rt + acc_row(lane, e);
                    const int col = v0 + 16 * ct + acc_col(lane);
                    ht[row * V + col] = hacc[rt][ct][e];
                }
    }
}

template <typename T, int K, int V, int C, int VT, bool PK>
static hipError_t launch_scan_t(const ScanLaunch& a) {
    const int64_t chains = a.N * a.H;
    const int64_t nblk = ((chains + 7) / 8) * 8 * (V / VT);
    hipLaunchKernelGGL((scan_kernel<T, K, V, C, VT, PK>), dim3((unsigned)nblk), dim3(256), 0,
                       a.stream, a);
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
    return a.bf16 ? launch_scan_dt<bf16, 32>(a) : launch_scan_dt<float, 16>(a);
}

}  // namespace gdn
