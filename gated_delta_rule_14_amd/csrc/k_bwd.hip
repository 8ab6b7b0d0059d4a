// Backward pass of the chunked gated delta rule (scalar gate, C = 64).
//
// "阅读笔记：DeltaNet 在 FLA 中的代码实现笔记" (二、反向传播) lays the backward out
// in six steps: recompute U, W (Step 1) and the chunk entry states (Step 2);
// the intra-chunk part of dU (Step 3); a reverse recurrence for the state
// gradient (Step 4); dQ, dK part 1, dW (Step 5); the WY backward for dV,
// dK part 2 and dbeta (Step 6).  The pages write it for the ungated DeltaNet;
// with the gate, per chunk of n <= C tokens (G the inclusive cumulative gate,
// gamma = 2^G in log2 units, Gamma_ij = gamma_i / gamma_j for j <= i,
// Ks = diag(gamma_C / gamma) K, Qs = scale diag(gamma) Q, T = (I + A)^{-1},
// h the state entering the chunk and dH the gradient of the one leaving it):
//   dVn  = Aqk^T dO + Ks dH                               (Steps 3-4)
//   dH  <- gamma_C dH + Qs^T dO - W^T dVn                  (Step 4)
//   dQ   = scale diag(gamma) dO h^T + Pm K,   Pm = scale (dO Vn^T) * Gamma (j <= i)
//   dK   = diag(gamma_C / gamma) Vn dH^T + Pm^T Q          (Step 5)
//        + diag(beta gamma) T^T dW + (Z + Z^T) K           (Step 6)
//   dV   = diag(beta) T^T dVn,  dW = -dVn h^T
//   dA   = -T^T (dVn (diag(beta) V)^T + dW (diag(beta gamma) K)^T) T^T,
//   Z    = diag(beta) (dA * Gamma)  (strictly lower)
//   dbeta_i = (T^T dVn)_i . v_i + gamma_i (T^T dW)_i . k_i + sum_j (dA * Gamma)_ij k_i . k_j
// and the gate, which the pages do not cover: the gradient dG_i of the
// cumulative gate collects every place where gamma_i, or a Gamma entry of
// row or column i, enters (the output's state term, Aqk and A by rows minus
// columns, W's diag(gamma), Ks, and gamma_C on the carried state and on Ks
// for the last row), and dg = the reverse cumulative sum of dG in the chunk.
//
// Two kernels here; the forward intra stage (backward mode) and the forward
// state pass (storing entry states and V_new) run before them:
//   bwd_scan_kernel   the reverse recurrence, serial over chunks, one
//                     workgroup per (sequence, head, 32-column value slice)
//   bwd_local_kernel  every per-chunk gradient, one workgroup per (chunk, head)
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

// =====================================================================
// Reverse state-gradient pass.  The mirror of the forward state pass: the
// carried dH (K x VT, fp32) lives in MFMA accumulators of the dH waves; the
// operands Ks, Aqk^T, Qs^T, W^T come from the intra stage in fragment order
// (one coalesced 16-byte load per lane, issued PD steps ahead); dO is staged
// row-major in LDS one chunk ahead and read with transposing loads.
//   dV waves (C/32): token rows 32m..32m+31 of dVn = Ks dH + Aqk^T dO
//   dH waves (K/32): key rows 32p..32p+31 of dH
//   one store wave: dH and dVn of every chunk to HBM in fragment order
// Per step: dV waves read dH^T, publish dVn^T and the next chunk's dO,
// barrier; dH waves add Qs^T dO (before it) and -W^T dVn (after it), decay,
// publish dH^T, barrier.  The store wave reads dH^T before the first barrier
// (still the gradient leaving the chunk) and dVn^T between the two.
// =====================================================================

constexpr int BSCAN_MAX_THREADS = 512;

template <typename T, int K_, int V_, int VT_, int PD_, bool PK_ = false>
struct BScanCfg {
    typedef T Elt;
    static constexpr bool PK = PK_;   // per-key gate: the carried dH decays row by row
    typedef Mma<T> M;
    typedef FragOrder<T> F;
    static constexpr int K = K_, V = V_, C = 64, VT = VT_, PD = PD_;
    static constexpr int KS = M::KSTEP, KG = F::KG, KSPG = KG / KS;
    static constexpr int CT = VT / 16;
    static constexpr int NVW = C / 32, NHW = K / 32, NW = NVW + NHW + 1, NT = 64 * NW;
    static constexpr int GK = K / KG, GC = C / KG;
    static constexpr int P = 16 / sizeof(T);
    static constexpr int LDH = K + P;      // dH^T   [VT][K]
    static constexpr int LDV = C + P;      // dVn^T  [VT][C]
    static constexpr int LDO = VT + P;     // dO     [C][VT], two buffers
    static constexpr int NPC = VT * (int)sizeof(T) / 16;   // 16-byte pieces per dO row
    static constexpr int PPL = 32 * NPC / 64;              // pieces per lane (32 rows a wave)
    static constexpr size_t o_hT = 0;
    static constexpr size_t o_Vn = o_hT + sizeof(T) * VT * LDH;
    static constexpr size_t o_dO = o_Vn + sizeof(T) * VT * LDV;
    static constexpr size_t bytes = o_dO + 2 * sizeof(T) * C * LDO;
    static_assert(NT <= BSCAN_MAX_THREADS && PPL >= 1, "shape");
};

template <typename Cfg>
struct BChain {
    typedef typename Cfg::Elt T;
    const BwdScanLaunch& a;
    T *shT, *sVn, *sdO;
    int64_t n, h, t0, len, c0;
    int v0, nch, lane;

    __device__ __forceinline__ BChain(const BwdScanLaunch& la, char* smem, int64_t chain, int vt)
        : a(la) {
        shT = reinterpret_cast<T*>(smem + Cfg::o_hT);
        sVn = reinterpret_cast<T*>(smem + Cfg::o_Vn);
        sdO = reinterpret_cast<T*>(smem + Cfg::o_dO);
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
        if (c0 + nch > a.map.max_chunks) nch = (int)max((int64_t)0, a.map.max_chunks - c0);
    }
    // chunk processed at step s (last chunk first), clamped into the chain
    __device__ __forceinline__ int chunk_of(int s) const { return max(nch - 1 - s, 0); }
    __device__ __forceinline__ int64_t blk(int j) const { return h * a.map.max_chunks + c0 + j; }
    __device__ __forceinline__ T* dO_buf(int s) const { return sdO + (s & 1) * Cfg::C * Cfg::LDO; }
    // B fragment (value tile ct, k-offset k0) from a transposed buffer X^T[VT][ld]
    __device__ __forceinline__ typename Cfg::M::frag lds_frag(const T* x, int ld, int ct,
                                                             int k0) const {
        return Cfg::M::load(x + (16 * ct + (lane & 15)) * ld + k0, lane);
    }
    // raw dO pieces of rows 32m.. of chunk j (zero past the sequence end)
    __device__ __forceinline__ void load_dO(u32x4* d, int m, int j, bool any) const {
        const T* dout = static_cast<const T*>(a.dout);
#pragma unroll
        for (int p = 0; p < Cfg::PPL; ++p) {
            const int i = lane + 64 * p, r = 32 * m + i / Cfg::NPC, cp = i % Cfg::NPC;
            const int64_t tok = (int64_t)j * Cfg::C + r;
            d[p] = u32x4{0u, 0u, 0u, 0u};
            if (any && tok < len)
                d[p] = *reinterpret_cast<const u32x4*>(dout + ((t0 + tok) * a.H + h) * Cfg::V + v0 +
                                                      cp * (16 / sizeof(T)));
        }
    }
    __device__ __forceinline__ void put_dO(const u32x4* d, int m, T* buf) const {
#pragma unroll
        for (int p = 0; p < Cfg::PPL; ++p) {
            const int i = lane + 64 * p, r = 32 * m + i / Cfg::NPC, cp = i % Cfg::NPC;
            *reinterpret_cast<u32x4*>(buf + r * Cfg::LDO + cp * (16 / sizeof(T))) = d[p];
        }
    }
};

// ---- dV waves: dVn rows 32m..32m+31, all VT columns
template <typename Cfg>
struct BScanDV {
    typedef typename Cfg::Elt T;
    typedef typename Cfg::M M;
    typedef typename Cfg::F F;
    static constexpr int K = Cfg::K, V = Cfg::V, C = Cfg::C, CT = Cfg::CT, GK = Cfg::GK,
                         GC = Cfg::GC;
    struct Pre {
        u32x4 ks[2][GK];
        u32x4 aq[2][GC];
        u32x4 dnext[Cfg::PPL];   // dO of the chunk of the following step
    };
    const BChain<Cfg>& ch;
    int m;

    __device__ __forceinline__ void issue(Pre& p, int s) const {
        const int64_t b = ch.blk(ch.chunk_of(s));
        const u32x4* gk = reinterpret_cast<const u32x4*>(static_cast<const T*>(ch.a.ksr) + b * C * K);
        const u32x4* ga = reinterpret_cast<const u32x4*>(static_cast<const T*>(ch.a.aqkt) + b * C * C);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int sg = 0; sg < GK; ++sg) p.ks[t][sg] = gk[((2 * m + t) * GK + sg) * 64 + ch.lane];
#pragma unroll
            for (int sg = 0; sg < GC; ++sg) p.aq[t][sg] = ga[((2 * m + t) * GC + sg) * 64 + ch.lane];
        }
        ch.load_dO(p.dnext, m, ch.nch - 2 - s, s + 1 < ch.nch);
    }

    // dO of the first step (the last chunk) into buffer 0
    __device__ __forceinline__ void init() const {
        u32x4 d[Cfg::PPL];
        ch.load_dO(d, m, ch.nch - 1, ch.nch > 0);
        ch.put_dO(d, m, ch.dO_buf(0));
    }

    __device__ __forceinline__ void step(int s, const Pre& cur, Pre& spare) const {
        issue(spare, s + Cfg::PD);
        const T* sdo = ch.dO_buf(s);
        f32x4 acc[2][CT];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) acc[t][ct] = zero4();
        // Ks dH
#pragma unroll
        for (int sg = 0; sg < GK; ++sg)
#pragma unroll
            for (int i = 0; i < Cfg::KSPG; ++i) {
                const int k0 = sg * Cfg::KG + i * Cfg::KS;
                const typename M::frag a0 = F::frag(cur.ks[0][sg], i);
                const typename M::frag a1 = F::frag(cur.ks[1][sg], i);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const typename M::frag bh = ch.lds_frag(ch.shT, Cfg::LDH, ct, k0);
                    acc[0][ct] = M::mma(a0, bh, acc[0][ct]);
                    acc[1][ct] = M::mma(a1, bh, acc[1][ct]);
                }
            }
        // + Aqk^T dO
#pragma unroll
        for (int sg = 0; sg < GC; ++sg)
#pragma unroll
            for (int i = 0; i < Cfg::KSPG; ++i) {
                const int k0 = sg * Cfg::KG + i * Cfg::KS;
                const typename M::frag a0 = F::frag(cur.aq[0][sg], i);
                const typename M::frag a1 = F::frag(cur.aq[1][sg], i);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const typename M::frag bo = M::load_t(sdo + k0 * Cfg::LDO + 16 * ct, Cfg::LDO, ch.lane);
                    acc[0][ct] = M::mma(a0, bo, acc[0][ct]);
                    acc[1][ct] = M::mma(a1, bo, acc[1][ct]);
                }
            }
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
                store_acc_t(ch.sVn + 16 * ct * Cfg::LDV + 16 * (2 * m + t), Cfg::LDV, ch.lane,
                            acc[t][ct]);
        // the other buffer was last read in the previous step
        ch.put_dO(cur.dnext, m, ch.dO_buf(s + 1));
        lds_barrier();   // dVn^T and the next dO published
        lds_barrier();   // next dH^T published
    }
};

// ---- dH waves: dH rows 32p..32p+31 (key tiles 2p, 2p+1), all VT columns
template <typename Cfg>
struct BScanDH {
    typedef typename Cfg::Elt T;
    typedef typename Cfg::M M;
    typedef typename Cfg::F F;
    static constexpr int K = Cfg::K, V = Cfg::V, C = Cfg::C, CT = Cfg::CT, GC = Cfg::GC;
    static constexpr bool PK = Cfg::PK;
    struct Pre {
        u32x4 qs[2][GC];
        u32x4 wt[2][GC];
        float d[PK ? 8 : 1];   // log2 chunk-end decay (per key row for the per-key gate)
    };
    const BChain<Cfg>& ch;
    int p;
    f32x4 hacc[2][CT];

    __device__ __forceinline__ int row(int r, int e) const {
        return 16 * (2 * p + r) + acc_row(ch.lane, e);
    }

    __device__ __forceinline__ void issue(Pre& q, int s) const {
        const int64_t b = ch.blk(ch.chunk_of(s));
        const u32x4* gq = reinterpret_cast<const u32x4*>(static_cast<const T*>(ch.a.qst) + b * C * K);
        const u32x4* gw = reinterpret_cast<const u32x4*>(static_cast<const T*>(ch.a.wt) + b * C * K);
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int sg = 0; sg < GC; ++sg) {
                q.qs[r][sg] = gq[((2 * p + r) * GC + sg) * 64 + ch.lane];
                q.wt[r][sg] = gw[((2 * p + r) * GC + sg) * 64 + ch.lane];
            }
        if (PK) {
            const float* gd = ch.a.gcum + (b * C + (C - 1)) * K;
#pragma unroll
            for (int r = 0; r < 2; ++r)
#pragma unroll
                for (int e = 0; e < 4; ++e) q.d[PK ? 4 * r + e : 0] = gd[row(r, e)];
        } else {
            q.d[0] = ch.a.gcum[b * C + (C - 1)];
        }
    }

    // dH <- dht (or 0); publish dH^T
    __device__ __forceinline__ void init() {
        const float* dht = ch.a.dht ? ch.a.dht + (ch.n * ch.a.H + ch.h) * (int64_t)(K * V) : nullptr;
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    hacc[r][ct][e] =
                        dht ? dht[row(r, e) * V + ch.v0 + 16 * ct + acc_col(ch.lane)] : 0.f;
                store_acc_t(ch.shT + 16 * ct * Cfg::LDH + 16 * (2 * p + r), Cfg::LDH, ch.lane,
                            hacc[r][ct]);
            }
    }

    __device__ __forceinline__ void step(int s, const Pre& cur, Pre& spare) {
        issue(spare, s + Cfg::PD);
        const T* sdo = ch.dO_buf(s);
        f32x4 acc[2][CT], neg[2][CT];
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) acc[r][ct] = neg[r][ct] = zero4();
        // Qs^T dO
#pragma unroll
        for (int sg = 0; sg < GC; ++sg)
#pragma unroll
            for (int i = 0; i < Cfg::KSPG; ++i) {
                const int k0 = sg * Cfg::KG + i * Cfg::KS;
                const typename M::frag a0 = F::frag(cur.qs[0][sg], i);
                const typename M::frag a1 = F::frag(cur.qs[1][sg], i);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const typename M::frag bo = M::load_t(sdo + k0 * Cfg::LDO + 16 * ct, Cfg::LDO, ch.lane);
                    acc[0][ct] = M::mma(a0, bo, acc[0][ct]);
                    acc[1][ct] = M::mma(a1, bo, acc[1][ct]);
                }
            }
        float dec[2][4];
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int e = 0; e < 4; ++e) dec[r][e] = exp2_hw(cur.d[PK ? 4 * r + e : 0]);
        lds_barrier();   // dVn^T published
        // W^T dVn
#pragma unroll
        for (int sg = 0; sg < GC; ++sg)
#pragma unroll
            for (int i = 0; i < Cfg::KSPG; ++i) {
                const int k0 = sg * Cfg::KG + i * Cfg::KS;
                const typename M::frag a0 = F::frag(cur.wt[0][sg], i);
                const typename M::frag a1 = F::frag(cur.wt[1][sg], i);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const typename M::frag bv = ch.lds_frag(ch.sVn, Cfg::LDV, ct, k0);
                    neg[0][ct] = M::mma(a0, bv, neg[0][ct]);
                    neg[1][ct] = M::mma(a1, bv, neg[1][ct]);
                }
            }
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    hacc[r][ct][e] = dec[r][e] * hacc[r][ct][e] + acc[r][ct][e] - neg[r][ct][e];
                store_acc_t(ch.shT + 16 * ct * Cfg::LDH + 16 * (2 * p + r), Cfg::LDH, ch.lane,
                            hacc[r][ct]);
            }
        lds_barrier();   // next dH^T published
    }

    __device__ __forceinline__ void finish() const {
        if (!ch.a.dh0) return;
        float* d0 = ch.a.dh0 + (ch.n * ch.a.H + ch.h) * (int64_t)(K * V);
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    d0[row(r, e) * V + ch.v0 + 16 * ct + acc_col(ch.lane)] = hacc[r][ct][e];
    }
};

// ---- the store wave
template <typename Cfg>
struct BScanStore {
    typedef typename Cfg::Elt T;
    static constexpr int K = Cfg::K, V = Cfg::V, C = Cfg::C;
    struct Pre {};
    const BChain<Cfg>& ch;
    __device__ __forceinline__ void issue(Pre&, int) const {}
    __device__ __forceinline__ void step(int s, const Pre&, Pre&) const {
        const int64_t b = ch.blk(ch.chunk_of(s));
        store_frag_groups<T, Cfg::VT>(ch.shT, Cfg::LDH, static_cast<T*>(ch.a.dhs) + b * K * V, V,
                                      ch.v0, 0, K / 16, ch.lane);
        lds_barrier();   // dVn^T published
        store_frag_groups<T, Cfg::VT>(ch.sVn, Cfg::LDV, static_cast<T*>(ch.a.dvn) + b * C * V, V,
                                      ch.v0, 0, C / 16, ch.lane);
        lds_barrier();   // next dH^T published
    }
};

template <typename Cfg>
__global__ __launch_bounds__(BSCAN_MAX_THREADS) void bwd_scan_kernel(BwdScanLaunch a) {
    __shared__ __attribute__((aligned(16))) char smem[Cfg::bytes];
    constexpr int NVT = Cfg::V / Cfg::VT;
    // the workgroups of one (sequence, head) share an id modulo 8: one XCD
    // and its L2 for the operands they all read
    const int64_t bid = blockIdx.x;
    const int vt = (int)((bid >> 3) % NVT);
    const int64_t chain = (bid & 7) + 8 * ((bid >> 3) / NVT);
    if (chain >= a.N * a.H) return;

    const BChain<Cfg> ch(a, smem, chain, vt);
    const int wave = wave_id();
    if (wave < Cfg::NVW) {
        BScanDV<Cfg> r{ch, wave};
        if (ch.nch > 0) {
            r.init();
            drive<Cfg::PD>(r, ch.nch);
        }
    } else if (wave < Cfg::NVW + Cfg::NHW) {
        BScanDH<Cfg> r{ch, wave - Cfg::NVW, {}};
        r.init();
        if (ch.nch > 0) drive<Cfg::PD>(r, ch.nch);
        r.finish();
    } else {
        BScanStore<Cfg> r{ch};
        if (ch.nch > 0) drive<Cfg::PD>(r, ch.nch);
    }
    drain_vmem();   // the prefetches past the first chunk
}

template <typename Cfg>
static hipError_t launch_bscan_cfg(const BwdScanLaunch& a) {
    const int64_t chains = a.N * a.H;
    const int64_t nblk = ((chains + 7) / 8) * 8 * (Cfg::V / Cfg::VT);
    hipLaunchKernelGGL((bwd_scan_kernel<Cfg>), dim3((unsigned)nblk), dim3(Cfg::NT), 0, a.stream, a);
    return hipGetLastError();
}

template <bool PK, int VT>
static hipError_t launch_bwd_scan_vt(const BwdScanLaunch& a) {
    if (a.K == 64 && a.V == 64) return launch_bscan_cfg<BScanCfg<bf16, 64, 64, VT, 2, PK>>(a);
    if (a.K == 64 && a.V == 128) return launch_bscan_cfg<BScanCfg<bf16, 64, 128, VT, 2, PK>>(a);
    if (a.K == 128 && a.V == 64) return launch_bscan_cfg<BScanCfg<bf16, 128, 64, VT, 2, PK>>(a);
    if (a.K == 128 && a.V == 128) return launch_bscan_cfg<BScanCfg<bf16, 128, 128, VT, 2, PK>>(a);
    return hipErrorInvalidValue;
}

template <bool PK>
static hipError_t launch_bwd_scan_g(const BwdScanLaunch& a) {
    if (!a.bf16) {   // the fp32 backward covers K = V = 64 (the per-chunk kernel's LDS)
        if (a.K == 64 && a.V == 64 && !PK) return launch_bscan_cfg<BScanCfg<float, 64, 64, 32, 1>>(a);
        return hipErrorInvalidValue;
    }
    // 16-wide value slices when even they give at most one workgroup per CU
    // (few long chains of unpacked input): the CUs the 32-wide ones would
    // leave idle share the state
    if (!a.map.seqs && a.N * a.H * (a.V / 16) <= 256) return launch_bwd_scan_vt<PK, 16>(a);
    return launch_bwd_scan_vt<PK, 32>(a);
}

hipError_t launch_bwd_scan(const BwdScanLaunch& a) {
    if (a.C != 64) return hipErrorInvalidValue;
    return a.per_key ? launch_bwd_scan_g<true>(a) : launch_bwd_scan_g<false>(a);
}

// =====================================================================
// Per-chunk gradients.  One 512-thread workgroup (8 waves) per (chunk,
// head), everything in LDS; the products, by phase:
//   A  dO h^T, Vn dH^T, -dVn h^T (C x K; h and dH fragments straight from
//      HBM, each loaded by one wave), dO Vn^T, Q K^T, K K^T (C x C)
//   B  Pm K, Pm^T Q, T^T dW (C x K), T^T dVn (C x V), dVn V^T, dW K^T (C x C)
//   C  Y = dAinv T^T
//   D  dA = -T^T Y, masked, gated, with the K K^T tile of phase A
//   E  (Z + Z^T) K
// A C x K (C x V) output tile stays in one wave's accumulators from phase A
// to its store.  Per-row sums (dbeta, dG) are reduced inside a wave and kept
// per wave in LDS, then summed over the waves.
// Rows past the chunk's n tokens are loaded as zero (and beta as 0), so they
// add nothing to any valid row; they are never stored.
// =====================================================================

constexpr int BLOCAL_THREADS = 512;

template <typename T, int K, int V>
struct LocalSmem {
    static constexpr int C = 64, NW = BLOCAL_THREADS / 64;
    // rows padded by 32 bytes (measured on the B=4, T=4096, H=16, d=128
    // backward: 16 bytes cost 10 us more per call, 48 bytes 5 us; the results
    // are the same)
    static constexpr int P = 32 / sizeof(T);
    static constexpr int LDK = K + P, LDV = V + P, LDC = C + P;
    static constexpr int LDX = (K > V ? K : V) + P;
    static constexpr int LDN = LDV > LDC ? LDV : LDC;
    static constexpr size_t o_Q = 0;
    static constexpr size_t o_K = o_Q + sizeof(T) * C * LDK;
    static constexpr size_t o_V = o_K + sizeof(T) * C * LDK;
    static constexpr size_t o_DVN = o_V + sizeof(T) * C * LDV;
    static constexpr size_t o_DO = o_DVN + sizeof(T) * C * LDV;   // dO [LDV], then dW [LDK]
    static constexpr size_t o_VN = o_DO + sizeof(T) * C * LDX;    // Vn [LDV], then T [LDC]
    static constexpr size_t o_PM = o_VN + sizeof(T) * C * LDN;    // Pm, then Y
    static constexpr size_t o_DA = o_PM + sizeof(T) * C * LDC;    // dAinv, then Z + Z^T
    static constexpr size_t o_G = o_DA + sizeof(T) * C * LDC;
    static constexpr size_t o_E = o_G + 4 * C;
    static constexpr size_t o_B = o_E + 4 * C;
    static constexpr size_t o_RB = o_B + 4 * C;                   // [NW][C] dbeta partials
    static constexpr size_t o_RG = o_RB + 4 * NW * C;             // [NW][C] dG partials
    static constexpr size_t bytes = o_RG + 4 * NW * C;
    static_assert(bytes <= 160 * 1024, "LDS");
};

// Inputs of one (chunk slot, head) item, held in registers from their loads
// to their LDS stores.
template <typename T, int K, int V>
struct LocalItem {
    static constexpr int C = 64, EV = 16 / sizeof(T), NW = BLOCAL_THREADS / 64;
    static constexpr int NKQ = C * K / EV / BLOCAL_THREADS;   // 16-byte pieces per thread
    static constexpr int NVV = C * V / EV / BLOCAL_THREADS;
    static constexpr int NG = V / FragOrder<T>::KG;
    static constexpr int NGW = (C / 16) * NG / NW;             // V_new groups per wave
    static_assert(NKQ * EV * BLOCAL_THREADS == C * K && NVV * EV * BLOCAL_THREADS == C * V &&
                      NGW * NW == (C / 16) * NG,
                  "whole pieces");
    int64_t t0, blk, h;
    int n;
    u32x4 q[NKQ], k[NKQ], v[NVV], o[NVV], vn[NGW], dvn[NGW], t[8 / EV];
    u32x4 hg[NG], dg[NG];
    float g, b;
};

template <typename T, int K, int V>
__global__ __launch_bounds__(BLOCAL_THREADS) void bwd_local_kernel(BwdLocalLaunch a) {
    typedef LocalSmem<T, K, V> L;
    typedef Mma<T> M;
    typedef typename M::frag Frag;
    constexpr int C = 64, NW = L::NW, KS = M::KSTEP, EV = 16 / sizeof(T);
    constexpr int LDK = L::LDK, LDV = L::LDV, LDC = L::LDC;
    constexpr int NKT = K / 16, NVT = V / 16;
    constexpr int TPK = NKT * (C / 16) / NW, TPV = NVT * (C / 16) / NW;
    static_assert(TPK >= 1 && TPV >= 1 && NW % NKT == 0 && NW % NVT == 0, "tile split");
    __shared__ __attribute__((aligned(16))) char smem[L::bytes];
    T *sQ, *sK, *sV, *sDVN, *sDO, *sDW, *sVN, *sT, *sPM, *sY, *sDA, *sS;
    float *sG, *sE, *sB, *sRB, *sRG;
    // (re)derived at the top of every item from an offset the compiler cannot
    // see is zero: the addresses are then computed where they are used
    // instead of being hoisted out of the item loop and held in registers
    auto bind_lds = [&](int zero) {
        char* m = smem + zero;
        sQ = reinterpret_cast<T*>(m + L::o_Q);
        sK = reinterpret_cast<T*>(m + L::o_K);
        sV = reinterpret_cast<T*>(m + L::o_V);
        sDVN = reinterpret_cast<T*>(m + L::o_DVN);
        sDO = reinterpret_cast<T*>(m + L::o_DO);
        sDW = sDO;
        sVN = reinterpret_cast<T*>(m + L::o_VN);
        sT = sVN;
        sPM = reinterpret_cast<T*>(m + L::o_PM);
        sY = sPM;
        sDA = reinterpret_cast<T*>(m + L::o_DA);
        sS = sDA;
        sG = reinterpret_cast<float*>(m + L::o_G);
        sE = reinterpret_cast<float*>(m + L::o_E);
        sB = reinterpret_cast<float*>(m + L::o_B);
        sRB = reinterpret_cast<float*>(m + L::o_RB);
        sRG = reinterpret_cast<float*>(m + L::o_RG);
    };

    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int64_t H = a.H, Hq = a.Hq > 0 ? a.Hq : a.H;

    // This wave's C x K output tiles: key tile kt and token tiles rtk[j].  They
    // are computed transposed (MFMA operands swapped), so lane l holds token
    // 16 rtk[j] + l%16 and its 4 consecutive keys kc .. kc+3: per-token sums
    // are in-lane plus two shuffles, and rows move as 8- (bf16) or 16-byte
    // vectors.  C x V tiles likewise.
    const int kt = wave % NKT, tl = lane & 15, kc = 16 * kt + 4 * (lane >> 4);
    int rtk[TPK];
#pragma unroll
    for (int j = 0; j < TPK; ++j) rtk[j] = wave / NKT + (NW / NKT) * j;
    typedef FragOrder<T> F;
    constexpr int NS = V / KS, NG = V / F::KG, KSPG = F::KG / KS;

    // The workgroup walks items (chunk slot, head) it, it + gridDim.x, ...;
    // the next item's h, dH and T (the loads phase A waits for longest) are
    // loaded into registers from phase C of the current one on (they are
    // dead by then); the other inputs are loaded at the top of its iteration.
    typedef LocalItem<T, K, V> Item;
    const int64_t items = a.map.max_chunks * H;
    auto decode = [&](int64_t it, Item& x) {
        const int64_t c = it / H;
        x.h = it - c * H;
        if (a.map.table) {
            const int4 e = a.map.table[c];
            x.t0 = e.x;
            x.n = e.y;
        } else {
            const int64_t b = c / a.map.nt, j = c - b * a.map.nt;
            x.t0 = b * a.map.T + j * C;
            x.n = (int)min((int64_t)C, a.map.T - j * C);
        }
        x.blk = x.h * a.map.max_chunks + c;
    };
    const u32x4 z = {0u, 0u, 0u, 0u};
    // h and dH rows of key tile kt (fragment-order groups, one coalesced
    // 16-byte load per lane each)
    // Every load below is unconditional and in bounds (clamped rows, values
    // past the end replaced by zero), so that each field is redefined on
    // every path and its registers are free between its uses.
    auto issue_state = [&](Item& x) {
        const u32x4* hsrc = reinterpret_cast<const u32x4*>(static_cast<const T*>(a.hs) + x.blk * K * V);
        const u32x4* dsrc = reinterpret_cast<const u32x4*>(static_cast<const T*>(a.dhs) + x.blk * K * V);
#pragma unroll
        for (int sg = 0; sg < NG; ++sg) {
            x.hg[sg] = hsrc[(kt * NG + sg) * 64 + lane];
            x.dg[sg] = dsrc[(kt * NG + sg) * 64 + lane];
        }
    };
    // everything else (rows >= n as zero)
    auto issue_small = [&](Item& x) {
        const T* ai = static_cast<const T*>(a.ainv) + x.blk * C * C + (tid / 8) * C + (tid % 8) * 8;
#pragma unroll
        for (int e = 0; e < 8 / EV; ++e) x.t[e] = *reinterpret_cast<const u32x4*>(ai + e * EV);
        const int rb = min(tid & (C - 1), max(x.n - 1, 0));
        x.g = a.gcum[x.blk * C + (tid & (C - 1))];
        float bv = a.beta[(x.t0 + rb) * H + x.h];
        if (a.act.flags & ACT_BETA_SIGMOID) bv = act_beta(bv, a.act.flags & ACT_BETA_NEG_EIG);
        x.b = (tid & (C - 1)) < x.n ? bv : 0.f;
    };
    auto issue_rest = [&](Item& x) {
        const T* q = static_cast<const T*>(a.q);
        const T* k = static_cast<const T*>(a.k);
        const T* v = static_cast<const T*>(a.v);
        const T* dout = static_cast<const T*>(a.dout);
        const int64_t hq = x.h / (H / Hq);   // grouped value heads: the shared q/k head
#pragma unroll
        for (int p = 0; p < Item::NKQ; ++p) {
            const int i = tid + BLOCAL_THREADS * p, r = i / (K / EV), cv = (i % (K / EV)) * EV;
            const int64_t g = ((x.t0 + r) * Hq + hq) * K + cv;
            x.q[p] = r < x.n ? *reinterpret_cast<const u32x4*>(q + g) : z;
            x.k[p] = r < x.n ? *reinterpret_cast<const u32x4*>(k + g) : z;
        }
#pragma unroll
        for (int p = 0; p < Item::NVV; ++p) {
            const int i = tid + BLOCAL_THREADS * p, r = i / (V / EV), cv = (i % (V / EV)) * EV;
            const int64_t g = ((x.t0 + r) * H + x.h) * V + cv;
            x.v[p] = r < x.n ? *reinterpret_cast<const u32x4*>(v + g) : z;
            x.o[p] = r < x.n ? *reinterpret_cast<const u32x4*>(dout + g) : z;
        }
        const u32x4* vn = reinterpret_cast<const u32x4*>(static_cast<const T*>(a.vn) + x.blk * C * V);
        const u32x4* dvn = reinterpret_cast<const u32x4*>(static_cast<const T*>(a.dvn) + x.blk * C * V);
#pragma unroll
        for (int p = 0; p < Item::NGW; ++p) {
            const int gi = wave + NW * p, r = 16 * (gi / NG) + tl;
            x.vn[p] = r < x.n ? vn[gi * 64 + lane] : z;
            x.dvn[p] = r < x.n ? dvn[gi * 64 + lane] : z;
        }
    };
    // the loaded inputs to LDS
    auto put = [&](const Item& x) {
        const bool l2 = a.act.flags & ACT_QK_L2NORM;   // a row is K / EV consecutive lanes
#pragma unroll
        for (int p = 0; p < Item::NKQ; ++p) {
            const int i = tid + BLOCAL_THREADS * p, r = i / (K / EV), cv = (i % (K / EV)) * EV;
            *reinterpret_cast<u32x4*>(sQ + r * LDK + cv) = l2 ? l2norm_piece<T, K / EV>(x.q[p]) : x.q[p];
            *reinterpret_cast<u32x4*>(sK + r * LDK + cv) = l2 ? l2norm_piece<T, K / EV>(x.k[p]) : x.k[p];
        }
#pragma unroll
        for (int p = 0; p < Item::NVV; ++p) {
            const int i = tid + BLOCAL_THREADS * p, r = i / (V / EV), cv = (i % (V / EV)) * EV;
            *reinterpret_cast<u32x4*>(sV + r * LDV + cv) = x.v[p];
            *reinterpret_cast<u32x4*>(sDO + r * LDV + cv) = x.o[p];
        }
        // V_new and its gradient: fragment-order groups to row-major LDS
#pragma unroll
        for (int p = 0; p < Item::NGW; ++p) {
            const int gi = wave + NW * p, r = 16 * (gi / NG) + tl, c0 = F::KG * (gi % NG);
            if constexpr (sizeof(T) == 2) {
                *reinterpret_cast<u32x4*>(sVN + r * LDV + c0 + F::col(lane, 0)) = x.vn[p];
                *reinterpret_cast<u32x4*>(sDVN + r * LDV + c0 + F::col(lane, 0)) = x.dvn[p];
            } else {
#pragma unroll
                for (int e = 0; e < F::VE; ++e) {
                    sVN[r * LDV + c0 + F::col(lane, e)] = __uint_as_float(x.vn[p][e]);
                    sDVN[r * LDV + c0 + F::col(lane, e)] = __uint_as_float(x.dvn[p][e]);
                }
            }
        }
        if (tid < C) {
            sG[tid] = x.g;
            sE[tid] = exp2_hw(x.g);
            sB[tid] = x.b;
        }
        for (int i = tid; i < 2 * NW * C; i += BLOCAL_THREADS) sRB[i] = 0.f;   // sRB, sRG
    };

    Item cur;
    int64_t it = blockIdx.x;
    decode(it, cur);
    issue_state(cur);
    issue_small(cur);
    while (it < items) {
    const int64_t itn = min(it + (int64_t)gridDim.x, items - 1);   // (the last one reloads)
    it += gridDim.x;
    if (cur.n <= 0) {   // an unused chunk slot (uniform over the workgroup)
        decode(itn, cur);
        issue_state(cur);
        issue_small(cur);
        continue;
    }
    int zero;
    asm volatile("s_mov_b32 %0, 0" : "=s"(zero));
    bind_lds(zero);
    const int64_t t0 = cur.t0, blk = cur.blk, h = cur.h;
    const int n = cur.n;
    issue_rest(cur);
    put(cur);
    lds_barrier();

    const float Gend = sG[C - 1];
    float* myRB = sRB + wave * C;
    float* myRG = sRG + wave * C;
    // C x C tile (rows 16 I + 4(l/16) + e, column 16 J + l%16): row sums,
    // added by the last lane of each row group
    auto add_rows = [&](float* dst, int r0, f32x4 x) {
        x = row_sum16(x);
        if ((lane & 15) == 15) {
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[r0 + acc_row(lane, e)] += x[e];
        }
    };
    // ... column sums (sign s), added by lanes 0..15
    auto add_cols = [&](float* dst, int c0, f32x4 x, float s) {
        const float y = sum_groups(x[0] + x[1] + x[2] + x[3]);
        if (lane < 16) dst[c0 + lane] += s * y;
    };
    // transposed tile of token tile r0: this lane's partial x of token r0 + l%16
    auto add_tok = [&](float* dst, int r0, float x) {
        x = sum_groups(x);
        if (lane < 16) dst[r0 + lane] += x;
    };

    // ================= phase A
    f32x4 dq[TPK], dk[TPK], dw[TPK];
    {
        f32x4 dks[TPK];
#pragma unroll
        for (int j = 0; j < TPK; ++j) dq[j] = dks[j] = dw[j] = zero4();
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const Frag bh = F::frag(cur.hg[s / KSPG], s % KSPG), bd = F::frag(cur.dg[s / KSPG], s % KSPG);
#pragma unroll
            for (int j = 0; j < TPK; ++j) {
                const int r = 16 * rtk[j] + tl;
                dq[j] = M::mma(bh, M::load(sDO + r * LDV + s * KS, lane), dq[j]);
                dks[j] = M::mma(bd, M::load(sVN + r * LDV + s * KS, lane), dks[j]);
                dw[j] = M::mma(bh, M::load(sDVN + r * LDV + s * KS, lane), dw[j]);
            }
        }
        // <dH, h>: each (key, value) element once, by the waves w < NKT
        float hd = 0.f;
        if (wave < NKT) {
#pragma unroll
            for (int sg = 0; sg < NG; ++sg)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (sizeof(T) == 2) {
                        hd += __uint_as_float(cur.hg[sg][e] << 16) * __uint_as_float(cur.dg[sg][e] << 16) +
                              __uint_as_float(cur.hg[sg][e] & 0xffff0000u) *
                                  __uint_as_float(cur.dg[sg][e] & 0xffff0000u);
                    } else {
                        hd += __uint_as_float(cur.hg[sg][e]) * __uint_as_float(cur.dg[sg][e]);
                    }
                }
        }
        hd = wave_sum(hd);
        // dQ's state term, dK's Ks term, and their gate terms
        float stot = 0.f;
#pragma unroll
        for (int j = 0; j < TPK; ++j) {
            const int r = 16 * rtk[j] + tl;
            const float gq = a.scale * sE[r], gk = exp2_hw(fminf(Gend - sG[r], 0.f));
            const f32x4 qv = Quad<T>::get(Quad<T>::load(sQ + r * LDK + kc));
            const f32x4 kv = Quad<T>::get(Quad<T>::load(sK + r * LDK + kc));
            float qd = 0.f, s_ = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dq[j][e] *= gq;
                dks[j][e] *= gk;
                qd += qv[e] * dq[j][e];
                s_ += kv[e] * dks[j][e];
            }
            add_tok(myRG, 16 * rtk[j], qd - s_);
            stot += s_;
            dk[j] = dks[j];
        }
        stot = wave_sum(stot);
        if (lane == 0) myRG[C - 1] += stot + exp2_hw(Gend) * hd;
    }
    // C x C tiles of this wave: (I, J) = divmod(LOWER[2 * wave + u], 4).  Only
    // the 10 tiles on and below the diagonal carry products (here and in
    // phase D); the table gives the SIMDs (waves w and w + 4) 3, 3, 2 and 2
    // of them, and the slots left over zero the 6 upper tiles of Pm.
    static_assert(NW == 8 && C == 64, "tile table");
    constexpr int LOWER[16] = {15, 10, 14, 5, 13, 1, 12, 2, 9, 3, 8, 6, 4, 7, 0, 11};
    f32x4 kk[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int id = LOWER[2 * wave + u], I = id / 4, J = id % 4;
        kk[u] = zero4();
        if (J > I) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                Elem<T>::store(sPM + (16 * I + acc_row(lane, e)) * LDC + 16 * J + acc_col(lane), 0.f);
            continue;
        }
        const f32x4 dqk = mma_tile<T>(sDO + 16 * I * LDV, LDV, sVN + 16 * J * LDV, LDV, V, lane, zero4());
        const f32x4 qk = mma_tile<T>(sQ + 16 * I * LDK, LDK, sK + 16 * J * LDK, LDK, K, lane, zero4());
        kk[u] = mma_tile<T>(sK + 16 * I * LDK, LDK, sK + 16 * J * LDK, LDK, K, lane, zero4());
        f32x4 pr;
        const int j = 16 * J + acc_col(lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * I + acc_row(lane, e);
            const float pm = j <= i ? a.scale * exp2_hw(fminf(sG[i] - sG[j], 0.f)) * dqk[e] : 0.f;
            Elem<T>::store(sPM + i * LDC + j, pm);
            pr[e] = pm * qk[e];
        }
        add_rows(myRG, 16 * I, pr);
        add_cols(myRG, 16 * J, pr, -1.f);
    }
    lds_barrier();   // dO and Vn are read: their regions take dW and T
#pragma unroll
    for (int j = 0; j < TPK; ++j) store4(sDW + (16 * rtk[j] + tl) * LDK + kc, -dw[j]);
#pragma unroll
    for (int e = 0; e < 8 / EV; ++e)
        *reinterpret_cast<u32x4*>(sT + (tid / 8) * LDC + (tid % 8) * 8 + e * EV) = cur.t[e];
    lds_barrier();

    // ================= phase B
    {
        f32x4 atdw[TPK];
#pragma unroll
        for (int j = 0; j < TPK; ++j) atdw[j] = zero4();
        // Pm and T are lower triangular: Pm K takes the tokens k <= r of its
        // row, Pm^T Q and T^T dW those k >= r, so a k step wholly on the
        // zero side of a token tile is skipped
#pragma unroll
        for (int k0 = 0; k0 < C; k0 += KS) {
            const Frag bk = M::load_t(sK + k0 * LDK + 16 * kt, LDK, lane);
            const Frag bq = M::load_t(sQ + k0 * LDK + 16 * kt, LDK, lane);
            const Frag bw = M::load_t(sDW + k0 * LDK + 16 * kt, LDK, lane);
#pragma unroll
            for (int j = 0; j < TPK; ++j) {
                const int r0 = 16 * (NW == NKT ? j : rtk[j]);   // every wave has all token tiles then
                if (k0 <= r0 + 15) dq[j] = M::mma(bk, M::load(sPM + (r0 + tl) * LDC + k0, lane), dq[j]);
                if (k0 + KS > r0) {
                    dk[j] = M::mma(bq, M::load_t(sPM + k0 * LDC + r0, LDC, lane), dk[j]);
                    atdw[j] = M::mma(bw, M::load_t(sT + k0 * LDC + r0, LDC, lane), atdw[j]);
                }
            }
        }
        T* gdq = static_cast<T*>(a.dq);
#pragma unroll
        for (int j = 0; j < TPK; ++j) {
            const int r = 16 * rtk[j] + tl;
            const float bg = sB[r] * sE[r];
            const f32x4 kv = Quad<T>::get(Quad<T>::load(sK + r * LDK + kc));
            float kx = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) kx += kv[e] * atdw[j][e];
            dk[j] += bg * atdw[j];
            add_tok(myRB, 16 * rtk[j], sE[r] * kx);
            add_tok(myRG, 16 * rtk[j], bg * kx);
            if (r < n) {
                if (a.dq_part)
                    *reinterpret_cast<f32x4*>(a.dq_part + ((t0 + r) * H + h) * K + kc) = dq[j];
                else
                    store4(gdq + ((t0 + r) * H + h) * K + kc, dq[j]);
            }
        }
    }
    {   // dV = diag(beta) T^T dVn (transposed tiles), and its dbeta term
        const int vt = wave % NVT, vc = 16 * vt + 4 * (lane >> 4);
        T* gdv = static_cast<T*>(a.dv);
#pragma unroll
        for (int j = 0; j < TPV; ++j) {
            const int r0 = 16 * (NW == NVT ? j : wave / NVT + (NW / NVT) * j), r = r0 + tl;
            f32x4 x = zero4();
#pragma unroll
            for (int k0 = 0; k0 < C; k0 += KS)
                if (k0 + KS > r0)   // T^T takes the tokens k >= r
                    x = M::mma(M::load_t(sDVN + k0 * LDV + 16 * vt, LDV, lane),
                               M::load_t(sT + k0 * LDC + r0, LDC, lane), x);
            const f32x4 vv = Quad<T>::get(Quad<T>::load(sV + r * LDV + vc));
            add_tok(myRB, r0, x[0] * vv[0] + x[1] * vv[1] + x[2] * vv[2] + x[3] * vv[3]);
            if (r < n) store4(gdv + ((t0 + r) * H + h) * V + vc, sB[r] * x);
        }
    }
    // dAinv = dVn (diag(beta) V)^T + dW (diag(beta gamma) K)^T: only its
    // tiles on and below the diagonal reach dA (below); the upper ones are
    // zeroed, as phase C multiplies them by zeros of T
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int id = LOWER[2 * wave + u], I = id / 4, J = id % 4;
        if (J > I) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                Elem<T>::store(sDA + (16 * I + acc_row(lane, e)) * LDC + 16 * J + acc_col(lane), 0.f);
            continue;
        }
        const f32x4 x1 = mma_tile<T>(sDVN + 16 * I * LDV, LDV, sV + 16 * J * LDV, LDV, V, lane, zero4());
        const f32x4 x2 = mma_tile<T>(sDW + 16 * I * LDK, LDK, sK + 16 * J * LDK, LDK, K, lane, zero4());
        const int j = 16 * J + acc_col(lane);
        const float bj = sB[j], bgj = sB[j] * sE[j];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            Elem<T>::store(sDA + (16 * I + acc_row(lane, e)) * LDC + j, bj * x1[e] + bgj * x2[e]);
    }
    lds_barrier();

    // the next item's h, dH and T, into this one's (dead) registers
    decode(itn, cur);
    issue_state(cur);
    issue_small(cur);

    // ================= phase C: Y = dAinv T^T, its tiles on and below the
    // diagonal (phase D reads no other); Y takes Pm's region, whose upper
    // tiles phase A zeroed.  T is lower triangular, so tile (I, J) takes
    // the k <= 16 J + 15 of dAinv's rows.
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int id = LOWER[2 * wave + u], I = id / 4, J = id % 4;
        if (J > I) continue;
        const f32x4 y = J < 2 ? mma_tile<T>(sDA + 16 * I * LDC, LDC, sT + 16 * J * LDC, LDC, 32, lane, zero4())
                              : mma_tile<T>(sDA + 16 * I * LDC, LDC, sT + 16 * J * LDC, LDC, C, lane, zero4());
        store_acc(sY + 16 * I * LDC + 16 * J, LDC, lane, y);
    }
    lds_barrier();

    // ================= phase D: dA = -T^T Y, strictly lower, gated (phase A's
    // tiles, whose K K^T each wave still holds)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int id = LOWER[2 * wave + u], I = id / 4, J = id % 4;
        if (J > I) continue;
        f32x4 x = zero4();
#pragma unroll
        for (int k0 = 0; k0 < C; k0 += KS)
            if (k0 + KS > 16 * I)   // T^T's rows i take the m >= i
                x = M::mma(M::load_t(sT + k0 * LDC + 16 * I, LDC, lane),
                           M::load_t(sY + k0 * LDC + 16 * J, LDC, lane), x);
        const int j = 16 * J + acc_col(lane);
        f32x4 rb, rr;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * I + acc_row(lane, e);
            const float dag = j < i ? -x[e] * exp2_hw(fminf(sG[i] - sG[j], 0.f)) : 0.f;
            const float z = sB[i] * dag;
            rb[e] = dag * kk[u][e];
            rr[e] = z * kk[u][e];
            // Z + Z^T, each position written once: (i, j) for j <= i, its
            // mirror (j, i) for j < i (on a diagonal tile the upper half
            // comes only from the mirrors)
            if (j <= i) Elem<T>::store(sS + i * LDC + j, z);
            if (j < i) Elem<T>::store(sS + j * LDC + i, z);
        }
        add_rows(myRB, 16 * I, rb);
        add_rows(myRG, 16 * I, rr);
        add_cols(myRG, 16 * J, rr, -1.f);
    }
    lds_barrier();

    // ================= phase E: dK += (Z + Z^T) K; stores
    {
#pragma unroll
        for (int k0 = 0; k0 < C; k0 += KS) {
            const Frag bk = M::load_t(sK + k0 * LDK + 16 * kt, LDK, lane);
#pragma unroll
            for (int j = 0; j < TPK; ++j)
                dk[j] = M::mma(bk, M::load(sS + (16 * rtk[j] + tl) * LDC + k0, lane), dk[j]);
        }
        T* gdk = static_cast<T*>(a.dk);
#pragma unroll
        for (int j = 0; j < TPK; ++j) {
            const int r = 16 * rtk[j] + tl;
            if (r < n) {
                if (a.dk_part)
                    *reinterpret_cast<f32x4*>(a.dk_part + ((t0 + r) * H + h) * K + kc) = dk[j];
                else
                    store4(gdk + ((t0 + r) * H + h) * K + kc, dk[j]);
            }
        }
    }
    lds_barrier();
    // dbeta and dg = reverse cumulative sum of dG over the chunk; with the
    // input activation, their chain rule to the raw logits
    if (wave == 0) {
        float db = 0.f, dG = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            db += sRB[w * C + lane];
            dG += sRG[w * C + lane];
        }
        const float rev = __shfl(dG, C - 1 - lane, 64);
        float suf = wave_incl_scan(rev, lane);   // at lane l: sum of dG[C-1-l ..]
        const int r = C - 1 - lane;
        if (a.act.flags & ACT_GATE) {
            // log alpha = -e^{A_log} softplus(x), x = a + dt_bias:
            // d/da = -e^{A_log} sigmoid(x), d/dA_log = log alpha
            const float araw = a.g[(t0 + min(r, n - 1)) * H + h];
            const float el = expf(a.act.A_log[h]), xa = araw + a.act.dt_bias[h];
            const float da = r < n ? -suf * el / (1.f + expf(-xa)) : 0.f;
            float pl = r < n ? -suf * el * softplus_f(xa) : 0.f, pd = da;
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) {
                pl += __shfl_xor(pl, off, 64);
                pd += __shfl_xor(pd, off, 64);
            }
            if (lane == 0) *reinterpret_cast<float2*>(a.act_part + 2 * blk) = make_float2(pl, pd);
            suf = da;
        }
        if (a.act.flags & ACT_BETA_SIGMOID) {
            // beta = m sigmoid(b): d/db = m sigmoid(b) sigmoid(-b)
            const float braw = a.beta[(t0 + min(lane, n - 1)) * H + h];
            const float m = (a.act.flags & ACT_BETA_NEG_EIG) ? 2.f : 1.f;
            db *= m / ((1.f + expf(-braw)) * (1.f + expf(braw)));
        }
        if (r < n) a.dg[(t0 + r) * H + h] = suf;
        if (lane < n) a.dbeta[(t0 + lane) * H + h] = db;
    }
    lds_barrier();   // LDS is free for the next item
    }
    drain_vmem();   // the last (unused) prefetch
}

// One persistent workgroup per workgroup slot of the device (as many per CU
// as the LDS allows), or one per item when there are fewer items.
static int device_cus() {
    static int cus = 0;
    if (!cus) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
            cus = n;
        else
            cus = 256;
    }
    return cus;
}

template <typename T, int K, int V>
static hipError_t launch_blocal_t(const BwdLocalLaunch& a) {
    const int64_t items = a.map.max_chunks * a.H;
    const int64_t per_cu = (int64_t)(160 * 1024 / LocalSmem<T, K, V>::bytes);
    const int64_t grid = min(items, (int64_t)device_cus() * per_cu);
    hipLaunchKernelGGL((bwd_local_kernel<T, K, V>), dim3((unsigned)grid), dim3(BLOCAL_THREADS), 0,
                       a.stream, a);
    return hipGetLastError();
}

hipError_t launch_bwd_local(const BwdLocalLaunch& a) {
    if (a.C != 64) return hipErrorInvalidValue;
    if (a.per_key) return launch_bwd_local_kda(a);
    if (!a.bf16) {
        // fp32 operands fit the LDS only at K = V = 64
        if (a.K == 64 && a.V == 64) return launch_blocal_t<float, 64, 64>(a);
        return hipErrorInvalidValue;
    }
    if (a.K == 64 && a.V == 64) return launch_blocal_t<bf16, 64, 64>(a);
    if (a.K == 64 && a.V == 128) return launch_blocal_t<bf16, 64, 128>(a);
    if (a.K == 128 && a.V == 64) return launch_blocal_t<bf16, 128, 64>(a);
    if (a.K == 128 && a.V == 128) return launch_blocal_t<bf16, 128, 128>(a);
    return hipErrorInvalidValue;
}

}  // namespace gdn

namespace gdn {

// dq (dk) of each q/k head: the sum of its value heads' fp32 terms, 4
// consecutive channels per thread (grouped value heads in the backward).
template <typename T>
__global__ __launch_bounds__(256) void gva_sum_kernel(GvaSumLaunch a) {
    const int64_t m = a.H / a.Hq, per_row = a.Hq * (a.K / 4);
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= a.rows * per_row) return;
    const int64_t row = i / per_row, rest = i - row * per_row;
    const int64_t hq = rest / (a.K / 4), c = (rest - hq * (a.K / 4)) * 4;
    f32x4 acc = zero4();
    for (int64_t u = 0; u < m; ++u)
        acc += *reinterpret_cast<const f32x4*>(a.part + (row * a.H + hq * m + u) * a.K + c);
    store4(static_cast<T*>(a.out) + (row * a.Hq + hq) * a.K + c, acc);
}

// dA_log[h] and ddt_bias[h]: one workgroup per head sums the per-chunk
// terms of the slots in use, in a fixed order (deterministic).
__global__ __launch_bounds__(256) void act_reduce_kernel(ActReduceLaunch a) {
    __shared__ float sl[256], sd[256];
    const int64_t h = blockIdx.x, mc = a.map.max_chunks;
    const int tid = threadIdx.x;
    float l = 0.f, d = 0.f;
    for (int64_t c = tid; c < mc; c += 256) {
        if (a.map.table && a.map.table[c].y <= 0) continue;
        const float2 p = *reinterpret_cast<const float2*>(a.part + 2 * (h * mc + c));
        l += p.x;
        d += p.y;
    }
    sl[tid] = l;
    sd[tid] = d;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
        if (tid < off) {
            sl[tid] += sl[tid + off];
            sd[tid] += sd[tid + off];
        }
        __syncthreads();
    }
    if (tid == 0) {
        a.dA_log[h] = sl[0];
        a.ddt_bias[h] = sd[0];
    }
}

// Per-key gate: thread u of head h's workgroup sums column u of the
// per-chunk terms over the used slots, in slot order (u = 0: dA_log[h];
// u = 2 + d: ddt_bias[h][d]).
__global__ __launch_bounds__(256) void act_reduce_pk_kernel(ActReduceLaunch a) {
    const int64_t h = blockIdx.x, mc = a.map.max_chunks;
    const int S = a.K + 2;
    for (int u = threadIdx.x; u < S; u += 256) {
        if (u == 1) continue;
        float s = 0.f;
        for (int64_t c = 0; c < mc; ++c) {
            if (a.map.table && a.map.table[c].y <= 0) continue;
            s += a.part[(h * mc + c) * S + u];
        }
        if (u == 0)
            a.dA_log[h] = s;
        else
            a.ddt_bias[h * a.K + (u - 2)] = s;
    }
}

hipError_t launch_act_reduce(const ActReduceLaunch& a) {
    if (a.H <= 0) return hipSuccess;
    if (a.K > 0)
        hipLaunchKernelGGL(act_reduce_pk_kernel, dim3((unsigned)a.H), dim3(256), 0, a.stream, a);
    else
        hipLaunchKernelGGL(act_reduce_kernel, dim3((unsigned)a.H), dim3(256), 0, a.stream, a);
    return hipGetLastError();
}

// dx = (dy - x (x.dy) / n2) / sqrt(n2) per row, in place over dy: 16-byte
// pieces, K / EV consecutive lanes per row.
template <typename T, int K>
__global__ __launch_bounds__(256) void l2norm_bwd_kernel(L2BwdLaunch a) {
    constexpr int EV = 16 / sizeof(T), LPR = K / EV;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const bool live = i < a.rows * LPR;
    const int64_t off = (live ? i : 0) * EV;   // idle lanes read piece 0 and store nothing
    const u32x4 xp = *reinterpret_cast<const u32x4*>(static_cast<const T*>(a.x) + off);
    const u32x4 dp = *reinterpret_cast<const u32x4*>(static_cast<const T*>(a.dx) + off);
    float x[EV], dy[EV];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if constexpr (sizeof(T) == 2) {
            x[2 * e] = __uint_as_float(xp[e] << 16);
            x[2 * e + 1] = __uint_as_float(xp[e] & 0xffff0000u);
            dy[2 * e] = __uint_as_float(dp[e] << 16);
            dy[2 * e + 1] = __uint_as_float(dp[e] & 0xffff0000u);
        } else {
            x[e] = __uint_as_float(xp[e]);
            dy[e] = __uint_as_float(dp[e]);
        }
    }
    float ss = 0.f, xd = 0.f;
#pragma unroll
    for (int e = 0; e < EV; ++e) {
        ss += x[e] * x[e];
        xd += x[e] * dy[e];
    }
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) {
        ss += __shfl_xor(ss, o, 64);
        xd += __shfl_xor(xd, o, 64);
    }
    const float n2 = ss + L2_EPS, c = xd / n2, inv = 1.f / sqrtf(n2);
    u32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if constexpr (sizeof(T) == 2)
            r[e] = pack_bf16x2((dy[2 * e] - x[2 * e] * c) * inv, (dy[2 * e + 1] - x[2 * e + 1] * c) * inv);
        else
            r[e] = __float_as_uint((dy[e] - x[e] * c) * inv);
    }
    if (live) *reinterpret_cast<u32x4*>(static_cast<T*>(a.dx) + off) = r;
}

hipError_t launch_l2norm_bwd(const L2BwdLaunch& a) {
    if (a.rows <= 0) return hipSuccess;
    const int ev = a.bf16 ? 8 : 4;
    const int64_t n = a.rows * (a.K / ev);
    const dim3 grid((unsigned)((n + 255) / 256));
    if (a.bf16 && a.K == 128)
        hipLaunchKernelGGL((l2norm_bwd_kernel<bf16, 128>), grid, dim3(256), 0, a.stream, a);
    else if (a.bf16 && a.K == 64)
        hipLaunchKernelGGL((l2norm_bwd_kernel<bf16, 64>), grid, dim3(256), 0, a.stream, a);
    else if (!a.bf16 && a.K == 128)
        hipLaunchKernelGGL((l2norm_bwd_kernel<float, 128>), grid, dim3(256), 0, a.stream, a);
    else if (!a.bf16 && a.K == 64)
        hipLaunchKernelGGL((l2norm_bwd_kernel<float, 64>), grid, dim3(256), 0, a.stream, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_gva_sum(const GvaSumLaunch& a) {
    const int64_t n = a.rows * a.Hq * (a.K / 4);
    if (n <= 0) return hipSuccess;
    const dim3 grid((unsigned)((n + 255) / 256));
    if (a.bf16)
        hipLaunchKernelGGL(gva_sum_kernel<bf16>, grid, dim3(256), 0, a.stream, a);
    else
        hipLaunchKernelGGL(gva_sum_kernel<float>, grid, dim3(256), 0, a.stream, a);
    return hipGetLastError();
}

}  // namespace gdn
