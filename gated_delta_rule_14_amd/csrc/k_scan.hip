// Inter-chunk state pass with the chunk output fused in (k4 + k5).
//
// The state h (K x V, fp32) is carried serially over the chunks of one
// (sequence, head); the value dimension is split into VT-wide slices that run
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
// Data path.  W, Qs, Ks^T and Aqk sit in the workspace in MFMA fragment order
// and U in accumulator order (gdn_device.hpp), so every operand fragment is
// one coalesced 16-byte load per lane straight into registers, issued PD
// chunks ahead of its use; no operand is staged through LDS.  LDS holds only
// the two values that cross waves: h^T (a T copy of the state) and V_new^T.
// Each operand fragment is loaded by exactly one wave of the workgroup:
//   V waves (C/32): token rows 32m..32m+31 of V_new = U - W h
//   O waves (C/32): token columns 32m.. of O^T = h^T Qs^T + V_new^T Aqk^T
//   H waves (K/32): key rows 32p..32p+31 of h, held in MFMA accumulators
// Per chunk: V and O waves read h^T, V waves publish V_new^T, barrier; O
// waves finish and store their rows of O, H waves decay and update h and
// publish h^T, barrier.
//
// For the backward pass the same walk runs without the output (o == nullptr)
// and its O waves store, per chunk, the state that enters it and V_new in
// fragment order ("阅读笔记：DeltaNet 在 FLA 中的代码实现笔记", backward
// Steps 1-2: the states and U, W are recomputed, not kept from the forward).
//
// The workgroups of one (sequence, head) get ids equal modulo 8, so the
// hardware's round-robin over the 8 XCDs puts them on one XCD and they share
// W, Qs, Ks and Aqk through its L2.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

constexpr int SCAN_MAX_THREADS = 512;

template <typename T, int K_, int V_, int C_, int VT_, bool PK_, int PD_>
struct ScanCfg {
    typedef T Elt;
    typedef Mma<T> M;
    typedef FragOrder<T> F;
    static constexpr int K = K_, V = V_, C = C_, VT = VT_, PD = PD_;
    static constexpr bool PK = PK_;
    static constexpr int KS = M::KSTEP, KG = F::KG, KSPG = KG / KS;
    static constexpr int CT = VT / 16;                 // value tiles of the slice
    static constexpr int NVW = C / 32, NOW = C / 32, NHW = K / 32;
    static constexpr int NW = NVW + NOW + NHW, NT = 64 * NW;
    static constexpr int GK = K / KG, GC = C / KG;    // fragment groups along K / C
    static constexpr int P = 16 / sizeof(T);
    static constexpr int LDH = K + P;                  // h^T     [VT][K]
    static constexpr int LDV = C + P;                  // V_new^T [VT][C]
    static constexpr size_t o_hT = 0;
    static constexpr size_t o_Vn = sizeof(T) * VT * LDH;
    static constexpr size_t bytes = o_Vn + sizeof(T) * VT * LDV;
    static_assert(C == 64, "two token pairs: the O waves are specialised for m = 0, 1");
    static_assert(K % 32 == 0 && VT % 16 == 0 && V % VT == 0, "tile shape");
    static_assert(NT <= SCAN_MAX_THREADS, "workgroup size");
    static_assert(PD >= 1 && PD <= 4, "prefetch distance");
};

// One (sequence, head, value slice): chunk range and shared pointers.
template <typename Cfg>
struct ScanChain {
    typedef typename Cfg::Elt T;
    const ScanLaunch& a;
    T* shT;
    T* sVn;
    int64_t n, h, t0, len, c0;
    int v0, nch, lane;

    __device__ __forceinline__ ScanChain(const ScanLaunch& la, char* smem, int64_t chain, int vt)
        : a(la) {
        shT = reinterpret_cast<T*>(smem + Cfg::o_hT);
        sVn = reinterpret_cast<T*>(smem + Cfg::o_Vn);
        const int64_t r = chain / a.H;   // packed input: longest sequence first
        n = a.map.seqs ? (int64_t)a.map.seqs[r].w : r;
        h = chain - r * a.H;
        v0 = vt * Cfg::VT;
        lane = threadIdx.x & 63;
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
        nch = (int)((len + Cfg::C - 1) / Cfg::C);
        // never walk past the chunk slots (only invalid offsets could ask to)
        if (c0 + nch > a.map.max_chunks) nch = (int)max((int64_t)0, a.map.max_chunks - c0);
    }
    // workspace block of chunk j (nch >= 1), clamped to the last chunk:
    // prefetches past the end reload it, so every step issues the same loads
    __device__ __forceinline__ int64_t blk(int j) const {
        return h * a.map.max_chunks + c0 + min(j, nch - 1);
    }
    // row r of the B operand read from a transposed LDS buffer X^T[VT][ld]:
    // the fragment for value tile ct and k-offset k0
    __device__ __forceinline__ typename Cfg::M::frag lds_frag(const T* x, int ld, int ct,
                                                             int k0) const {
        return Cfg::M::load(x + (16 * ct + (lane & 15)) * ld + k0, lane);
    }
};

// ---- V waves: V_new rows 32m..32m+31 (token tiles 2m, 2m+1), all VT columns
template <typename Cfg>
struct ScanV {
    typedef typename Cfg::Elt T;
    typedef typename Cfg::M M;
    typedef typename Cfg::F F;
    static constexpr int K = Cfg::K, V = Cfg::V, C = Cfg::C, CT = Cfg::CT, GK = Cfg::GK;
    struct Pre {
        u32x4 w[2][GK];
        typename Quad<T>::raw u[2][CT];
    };
    const ScanChain<Cfg>& ch;
    int m;

    __device__ __forceinline__ void issue(Pre& p, int j) const {
        const int64_t b = ch.blk(j);
        const u32x4* gw = reinterpret_cast<const u32x4*>(static_cast<const T*>(ch.a.ws.w) + b * C * K);
        const T* gu = static_cast<const T*>(ch.a.ws.u) + b * C * V;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int sg = 0; sg < GK; ++sg) p.w[t][sg] = gw[((2 * m + t) * GK + sg) * 64 + ch.lane];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
                p.u[t][ct] = Quad<T>::load(
                    gu + ((int64_t)((2 * m + t) * (V / 16) + ch.v0 / 16 + ct) * 64 + ch.lane) * 4);
    }

    __device__ __forceinline__ void step(int j, const Pre& cur, Pre& spare) const {
        issue(spare, j + Cfg::PD);
        f32x4 acc[2][CT];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) acc[t][ct] = zero4();
#pragma unroll
        for (int sg = 0; sg < GK; ++sg)
#pragma unroll
            for (int i = 0; i < Cfg::KSPG; ++i) {
                const int k0 = sg * Cfg::KG + i * Cfg::KS;
                const typename M::frag a0 = F::frag(cur.w[0][sg], i);
                const typename M::frag a1 = F::frag(cur.w[1][sg], i);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const typename M::frag bh = ch.lds_frag(ch.shT, Cfg::LDH, ct, k0);
                    acc[0][ct] = M::mma(a0, bh, acc[0][ct]);
                    acc[1][ct] = M::mma(a1, bh, acc[1][ct]);
                }
            }
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const f32x4 u = Quad<T>::get(cur.u[t][ct]);
                store_acc_t(ch.sVn + 16 * ct * Cfg::LDV + 16 * (2 * m + t), Cfg::LDV, ch.lane,
                            u - acc[t][ct]);
            }
        lds_barrier();   // V_new^T published
        lds_barrier();   // next h^T published
    }
};

// ---- O waves: O^T for token tiles 2M, 2M+1 (columns), all VT rows
template <typename Cfg, int MT>
struct ScanO {
    typedef typename Cfg::Elt T;
    typedef typename Cfg::M M;
    typedef typename Cfg::F F;
    static constexpr int K = Cfg::K, V = Cfg::V, C = Cfg::C, CT = Cfg::CT, GK = Cfg::GK;
    // Aqk groups along j that can be nonzero for tokens < 32(MT+1)
    static constexpr int NA = (32 * (MT + 1) + Cfg::KG - 1) / Cfg::KG;
    struct Pre {
        u32x4 q[2][GK];
        u32x4 a[2][NA];
    };
    const ScanChain<Cfg>& ch;

    __device__ __forceinline__ void issue(Pre& p, int j) const {
        const int64_t b = ch.blk(j);
        const u32x4* gq = reinterpret_cast<const u32x4*>(static_cast<const T*>(ch.a.ws.qs) + b * C * K);
        const u32x4* ga = reinterpret_cast<const u32x4*>(static_cast<const T*>(ch.a.ws.aqk) + b * C * C);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int sg = 0; sg < GK; ++sg) p.q[t][sg] = gq[((2 * MT + t) * GK + sg) * 64 + ch.lane];
#pragma unroll
            for (int sg = 0; sg < NA; ++sg)
                p.a[t][sg] = ga[((2 * MT + t) * Cfg::GC + sg) * 64 + ch.lane];
        }
    }

    __device__ __forceinline__ void step(int j, const Pre& cur, Pre& spare) const {
        issue(spare, j + Cfg::PD);
        f32x4 acc[CT][2];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) acc[ct][0] = acc[ct][1] = zero4();
        // h^T Qs^T: the entering state
#pragma unroll
        for (int sg = 0; sg < GK; ++sg)
#pragma unroll
            for (int i = 0; i < Cfg::KSPG; ++i) {
                const int k0 = sg * Cfg::KG + i * Cfg::KS;
                const typename M::frag b0 = F::frag(cur.q[0][sg], i);
                const typename M::frag b1 = F::frag(cur.q[1][sg], i);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const typename M::frag ah = ch.lds_frag(ch.shT, Cfg::LDH, ct, k0);
                    acc[ct][0] = M::mma(ah, b0, acc[ct][0]);
                    acc[ct][1] = M::mma(ah, b1, acc[ct][1]);
                }
            }
        lds_barrier();   // V_new^T published
        // + V_new^T Aqk^T (Aqk is zero above the diagonal)
#pragma unroll
        for (int sg = 0; sg < NA; ++sg)
#pragma unroll
            for (int i = 0; i < Cfg::KSPG; ++i) {
                const int k0 = sg * Cfg::KG + i * Cfg::KS;
                const typename M::frag b0 = F::frag(cur.a[0][sg], i);
                const typename M::frag b1 = F::frag(cur.a[1][sg], i);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const typename M::frag av = ch.lds_frag(ch.sVn, Cfg::LDV, ct, k0);
                    acc[ct][0] = M::mma(av, b0, acc[ct][0]);
                    acc[ct][1] = M::mma(av, b1, acc[ct][1]);
                }
            }
        // lane: 4 consecutive values of one token row of O
        const int ntok = (int)min((int64_t)C, ch.len - (int64_t)j * C);
        const int64_t tt0 = ch.t0 + (int64_t)j * C;
        T* o = static_cast<T*>(ch.a.o);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int tok = 16 * (2 * MT + t) + acc_col(ch.lane);
            if (tok < ntok) {
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
                    store4(o + ((tt0 + tok) * ch.a.H + ch.h) * V + ch.v0 + 16 * ct +
                               4 * (ch.lane >> 4),
                           acc[ct][t]);
            }
        }
        lds_barrier();   // next h^T published
    }
};

// ---- H waves: h rows 32p..32p+31 (key tiles 2p, 2p+1), all VT columns
template <typename Cfg>
struct ScanH {
    typedef typename Cfg::Elt T;
    typedef typename Cfg::M M;
    typedef typename Cfg::F F;
    static constexpr int K = Cfg::K, V = Cfg::V, C = Cfg::C, CT = Cfg::CT, GC = Cfg::GC;
    static constexpr bool PK = Cfg::PK;
    struct Pre {
        u32x4 k[2][GC];
        float d[PK ? 8 : 1];   // log2 chunk-end decay (per key row for the per-key gate)
    };
    const ScanChain<Cfg>& ch;
    int p;
    f32x4 hacc[2][CT];

    __device__ __forceinline__ int row(int r, int e) const {
        return 16 * (2 * p + r) + acc_row(ch.lane, e);
    }

    __device__ __forceinline__ void issue(Pre& q, int j) const {
        const int64_t b = ch.blk(j);
        const u32x4* gk = reinterpret_cast<const u32x4*>(static_cast<const T*>(ch.a.ws.ks) + b * C * K);
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int sg = 0; sg < GC; ++sg) q.k[r][sg] = gk[((2 * p + r) * GC + sg) * 64 + ch.lane];
        if (PK) {
            const float* gd = ch.a.ws.gcum + (b * C + (C - 1)) * K;
#pragma unroll
            for (int r = 0; r < 2; ++r)
#pragma unroll
                for (int e = 0; e < 4; ++e) q.d[(PK ? 4 * r + e : 0)] = gd[row(r, e)];
        } else {
            q.d[0] = ch.a.ws.gcum[b * C + (C - 1)];
        }
    }

    // h <- h0 (or 0); publish h^T
    __device__ __forceinline__ void init() {
        const float* h0 = ch.a.h0 ? ch.a.h0 + (ch.n * ch.a.H + ch.h) * (int64_t)(K * V) : nullptr;
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    hacc[r][ct][e] =
                        h0 ? h0[row(r, e) * V + ch.v0 + 16 * ct + acc_col(ch.lane)] : 0.f;
                store_acc_t(ch.shT + 16 * ct * Cfg::LDH + 16 * (2 * p + r), Cfg::LDH, ch.lane,
                            hacc[r][ct]);
            }
    }

    __device__ __forceinline__ void step(int j, const Pre& cur, Pre& spare) {
        issue(spare, j + Cfg::PD);
        float dec[2][4];
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int e = 0; e < 4; ++e) dec[r][e] = exp2_hw(cur.d[PK ? 4 * r + e : 0]);
        lds_barrier();   // V_new^T published
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) hacc[r][ct][e] *= dec[r][e];
#pragma unroll
        for (int sg = 0; sg < GC; ++sg)
#pragma unroll
            for (int i = 0; i < Cfg::KSPG; ++i) {
                const int k0 = sg * Cfg::KG + i * Cfg::KS;
                const typename M::frag a0 = F::frag(cur.k[0][sg], i);
                const typename M::frag a1 = F::frag(cur.k[1][sg], i);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const typename M::frag bv = ch.lds_frag(ch.sVn, Cfg::LDV, ct, k0);
                    hacc[0][ct] = M::mma(a0, bv, hacc[0][ct]);
                    hacc[1][ct] = M::mma(a1, bv, hacc[1][ct]);
                }
            }
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
                store_acc_t(ch.shT + 16 * ct * Cfg::LDH + 16 * (2 * p + r), Cfg::LDH, ch.lane,
                            hacc[r][ct]);
        lds_barrier();   // next h^T published
    }

    __device__ __forceinline__ void finish() const {
        if (!ch.a.ht) return;
        float* ht = ch.a.ht + (ch.n * ch.a.H + ch.h) * (int64_t)(K * V);
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    ht[row(r, e) * V + ch.v0 + 16 * ct + acc_col(ch.lane)] = hacc[r][ct][e];
    }
};

// ---- O waves of a walk without output: they store, per chunk, the state
// entering it (read from h^T in LDS before the step's first barrier, while
// it is still the entering state) and V_new (read from V_new^T after it), in
// fragment order, half of the row tiles each; or only keep the barriers.
template <typename Cfg>
struct ScanStore {
    typedef typename Cfg::Elt T;
    static constexpr int K = Cfg::K, V = Cfg::V, C = Cfg::C;
    struct Pre {};
    const ScanChain<Cfg>& ch;
    int w;   // 0 or 1
    __device__ __forceinline__ void issue(Pre&, int) const {}
    __device__ __forceinline__ void step(int j, const Pre&, Pre&) const {
        constexpr bool whole = Cfg::VT % FragOrder<T>::KG == 0 || (sizeof(T) == 2 && Cfg::VT == 16);
        if constexpr (whole) {
            if (ch.a.hs)
                store_frag_groups<T, Cfg::VT>(ch.shT, Cfg::LDH, static_cast<T*>(ch.a.hs) + ch.blk(j) * K * V,
                                              V, ch.v0, w * (K / 32), K / 32, ch.lane);
        }
        lds_barrier();   // V_new^T published
        if constexpr (whole) {
            if (ch.a.vn)
                store_frag_groups<T, Cfg::VT>(ch.sVn, Cfg::LDV, static_cast<T*>(ch.a.vn) + ch.blk(j) * C * V,
                                              V, ch.v0, w * (C / 32), C / 32, ch.lane);
        }
        lds_barrier();   // next h^T published
    }
};

template <typename Cfg>
__global__ __launch_bounds__(SCAN_MAX_THREADS) void scan_kernel(ScanLaunch a) {
    __shared__ __attribute__((aligned(16))) char smem[Cfg::bytes];
    constexpr int NVT = Cfg::V / Cfg::VT;
    const int64_t bid = blockIdx.x;
    const int vt = (int)((bid >> 3) % NVT);
    const int64_t chain = (bid & 7) + 8 * ((bid >> 3) / NVT);
    if (chain >= a.N * a.H) return;

    const ScanChain<Cfg> ch(a, smem, chain, vt);
    const int wave = wave_id();
    if (wave < Cfg::NVW) {
        ScanV<Cfg> r{ch, wave};
        if (ch.nch > 0) drive<Cfg::PD>(r, ch.nch);
    } else if (wave < Cfg::NVW + Cfg::NOW && !a.o) {
        ScanStore<Cfg> r{ch, wave - Cfg::NVW};
        if (ch.nch > 0) drive<Cfg::PD>(r, ch.nch);
    } else if (wave == Cfg::NVW) {
        ScanO<Cfg, 0> r{ch};
        if (ch.nch > 0) drive<Cfg::PD>(r, ch.nch);
    } else if (wave == Cfg::NVW + 1) {
        ScanO<Cfg, 1> r{ch};
        if (ch.nch > 0) drive<Cfg::PD>(r, ch.nch);
    } else {
        ScanH<Cfg> r{ch, wave - Cfg::NVW - Cfg::NOW, {}};
        r.init();
        if (ch.nch > 0) drive<Cfg::PD>(r, ch.nch);
        r.finish();
    }
    drain_vmem();   // the prefetches past the last chunk
}

template <typename Cfg>
static hipError_t launch_scan_cfg(const ScanLaunch& a) {
    const int64_t chains = a.N * a.H;
    const int64_t nblk = ((chains + 7) / 8) * 8 * (Cfg::V / Cfg::VT);
    hipLaunchKernelGGL((scan_kernel<Cfg>), dim3((unsigned)nblk), dim3(Cfg::NT), 0, a.stream, a);
    return hipGetLastError();
}

// value-slice width: one workgroup per CU when the chains allow it, and the
// narrowest slices for packed sequences (whose longest chain sets the time)
// (bf16 slices are at most 64 wide with K = 128: 128 would spill registers)
static int scan_vt(const ScanLaunch& a, bool bf16) {
    if (!bf16) return 32;
    // 16-wide slices when even they give at most one workgroup per CU (few
    // long chains; with the backward's per-chunk stores too, which then
    // write half fragment groups)
    if (!a.map.seqs && a.N * a.H * (a.V / 16) <= 256) return 16;
    const int min_nvt = (a.K == 128 && a.V == 128) ? 2 : 1;
    int nvt = a.V / 32;
    if (!a.map.seqs)
        while (nvt > min_nvt && a.N * a.H * nvt > 256) nvt /= 2;
    return a.V / nvt;
}

// prefetch distance (chunks) of the 32-wide bf16 slices
#ifndef GDN_SCAN_PD
#define GDN_SCAN_PD 2
#endif

template <typename T, int K, int V, bool PK>
static hipError_t launch_scan_kv(const ScanLaunch& a, int vt) {
    constexpr bool B = sizeof(T) == 2;
    if (vt == 32) return launch_scan_cfg<ScanCfg<T, K, V, 64, 32, PK, B ? GDN_SCAN_PD : 1>>(a);
    if constexpr (B) {
        if (vt == 16) return launch_scan_cfg<ScanCfg<T, K, V, 64, 16, PK, 2>>(a);
        if (vt == 64) return launch_scan_cfg<ScanCfg<T, K, V, 64, 64, PK, 2>>(a);
        if constexpr (V == 128 && K == 64)
            if (vt == 128) return launch_scan_cfg<ScanCfg<T, K, V, 64, 128, PK, 1>>(a);
    }
    return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_scan_dt(const ScanLaunch& a) {
    const int vt = scan_vt(a, sizeof(T) == 2);
#define GDN_SCAN_CASE(KK, VV)                                                         \
    if (a.K == KK && a.V == VV)                                                       \
        return a.per_key ? launch_scan_kv<T, KK, VV, true>(a, vt)                     \
                         : launch_scan_kv<T, KK, VV, false>(a, vt);
    GDN_SCAN_CASE(64, 64)
    GDN_SCAN_CASE(64, 128)
    GDN_SCAN_CASE(128, 64)
    GDN_SCAN_CASE(128, 128)
#undef GDN_SCAN_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_scan(const ScanLaunch& a) {
    if (a.C != 64) return hipErrorInvalidValue;
    return a.bf16 ? launch_scan_dt<bf16>(a) : launch_scan_dt<float>(a);
}

}  // namespace gdn
