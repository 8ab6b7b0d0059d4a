// Fused chunked forward: the intra-chunk products and the inter-chunk state
// pass in one kernel, for bf16 q/k/v with the scalar gate and K = V = 128.
//
// One workgroup (8 waves) per (sequence, head, 32-wide value slice) walks the
// chunks of its sequence in order.  Everything a chunk needs besides the state
// -- the cumulative gate, the masked products and the unit-lower inverse -- is
// built in LDS a step ahead of the state pass that consumes it, so no
// intermediate ever goes to HBM: the kernel reads q, k, v, beta, g and h0 once
// and writes o and ht once.
//
// Per chunk of n <= C = 64 tokens (rows r), with G the inclusive cumulative
// log2-gate inside the chunk and gamma_r = 2^{G_r} ("TileLang 实战：KDA 从零到一--
// Gated DeltaNet" §2.3 eqs. 11-12 and §4.1; "Gated Delta Network（GDN）"
// §4.1(a)-(d)):
//   A_ij   = beta_i 2^{G_i - G_j} k_i.k_j       (j < i)
//   T      = (I + A)^{-1}
//   Aqk_ij = scale 2^{G_i - G_j} q_i.k_j       (j <= i)
//   R      = diag(beta) (V - diag(gamma) K h)
//   V_new  = T R
//   O      = diag(scale gamma) Q h + Aqk V_new
//   h     <- gamma_C h + K^T diag(gamma_C / gamma) V_new
// T R equals the pages' U - W h with W = T diag(beta gamma) K and
// U = T diag(beta) V ("TileLang 实战" §2.2.4-2.2.6): the same product taken
// in the other order, so W and U are never formed.  The output reads the
// state entering the chunk; h is decayed before the chunk's contributions are
// added ("TileLang 实战" §4.4).
//
// The inverse: the four 16x16 diagonal blocks of I + A by forward
// substitution in fp32 (one wave, one lane per column), then the off-diagonal
// blocks from T_IJ = -T_II sum_{m=J}^{I-1} A_Im T_mJ on bf16 MFMA
// ("阅读笔记：DeltaNet 在 FLA 中的代码实现笔记", forward Step 2: 16x16 blocks
// solved first and combined block-wise; "TileLang 实战" §4.2).
//
// Schedule.  Iteration j runs the state pass of chunk j and builds the
// inverse of chunk j+1, in three phases separated by workgroup barriers:
//   P1  V waves: K h and R; O waves: Q h; H waves: decay h, diagonal K K^T
//       blocks of chunk j+1
//   P2  V waves: V_new = T R; O waves: the causal Q K^T blocks; H waves:
//       forward substitution and off-diagonal K K^T blocks of chunk j+1
//   P3  O waves: + Aqk V_new, store O; H waves: update h; V waves: compose the
//       off-diagonal blocks of chunk j+1's inverse
// Wave roles: waves 0-1 own token rows 32m..32m+31 of R and V_new, waves 2-3
// the token blocks {0, 3} and {1, 2} of O, waves 4-7 key rows 32p..32p+31 of h
// (fp32, in MFMA accumulators).  Chunk inputs arrive through registers loaded
// PD iterations ahead; K has three LDS slots and T two.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {
namespace fz {

constexpr int C = 64, K = 128, V = 128, VT = 32, CT = VT / 16, NVT = V / VT;
constexpr int NW = 8, NT = 64 * NW, PD = 2;
// Row pitches: 16-byte fragment reads from rows 288 or 160 bytes apart are
// free of LDS bank conflicts on gfx950, rows 272 or 144 bytes apart are not;
// transposing reads are conflict-free at either.
constexpr int LDK = K + 16;    // bf16 [C][LDK]    K, Q rows (288 B)
constexpr int LDVS = VT + 16;  // bf16 [C][LDVS]   V slice rows (transposing reads)
constexpr int LDA = 56;        // bf16 [48][LDA]   A rows 16..63, columns 0..47
constexpr int LDT = C + 8;     // fp32 [C][LDT]    T (288 B)
constexpr int LDN = 20;        // fp32 [4][NBS]    diagonal blocks of A, transposed
constexpr int NBS = 16 * LDN + 4;   // block stride: the four blocks start on different banks
constexpr int LDH = K + 16;    // bf16 [VT][LDH]   h^T (288 B)
constexpr int LDVN = C + 16;   // bf16 [VT][LDVN]  R^T, V_new^T, (V_new scaled)^T (160 B)
constexpr int NGA = 10;        // gate arrays per chunk slot
// Per token r of a chunk: G_LOG the cumulative log2 gate G_r; G_BETA beta_r;
// G_OUT scale 2^{G_r}; G_TAIL 2^{G_C - G_r}; G_GAM 2^{G_r}; G_END 2^{G_C}
// (every entry); G_ROW 2^{G_r - G_b}, b the first token of r's 16-token block;
// G_COL + I - 1 (I = 1, 2, 3): 2^{G_16I - G_r} for tokens r < 16I.
// Off-diagonal 16x16 blocks take their decay 2^{G_i - G_j} as
// G_ROW[i] * G_COL[I][j]: both factors lie in [0, 1], so neither overflows.
enum { G_LOG = 0, G_BETA = 1, G_OUT = 2, G_TAIL = 3, G_GAM = 4, G_END = 5, G_ROW = 6, G_COL = 7 };

constexpr size_t SZ_KQ = sizeof(bf16) * C * LDK;
constexpr size_t SZ_T = sizeof(float) * C * LDT;
constexpr size_t SZ_VN = sizeof(bf16) * VT * LDVN;
constexpr size_t o_K = 0;                                     // 3 slots
constexpr size_t o_Q = o_K + 3 * SZ_KQ;
constexpr size_t o_V = o_Q + SZ_KQ;
constexpr size_t o_A = o_V + sizeof(bf16) * C * LDVS;
constexpr size_t o_N = o_A + sizeof(bf16) * 48 * LDA;
constexpr size_t o_T = o_N + sizeof(float) * 4 * NBS;         // 2 slots
constexpr size_t o_hT = o_T + 2 * SZ_T;
constexpr size_t o_R = o_hT + sizeof(bf16) * VT * LDH;
constexpr size_t o_Vn = o_R + SZ_VN;
constexpr size_t o_Vt = o_Vn + SZ_VN;
constexpr size_t o_Gt = o_Vt + SZ_VN;
constexpr size_t BYTES = o_Gt + sizeof(float) * 3 * NGA * C;
static_assert(BYTES <= 160 * 1024, "LDS budget of one workgroup");
static_assert(o_A % 16 == 0 && o_N % 16 == 0 && o_T % 16 == 0 && o_hT % 16 == 0 &&
                  o_R % 16 == 0 && o_Gt % 16 == 0,
              "alignment");

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef Mma<bf16> M;

__device__ __forceinline__ f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x4 to_bf4(f32x4 v) {
    return __builtin_bit_cast(bf16x4, u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])});
}
// 16x16x16 A operand of a 16x16 block at `p` (row-major): lane 16g+m holds
// X[m][4g..4g+3]
__device__ __forceinline__ bf16x4 frag_a16(const float* p, int ld, int lane) {
    const float4 x = *reinterpret_cast<const float4*>(p + (lane & 15) * ld + 4 * (lane >> 4));
    return to_bf4(f32x4{x.x, x.y, x.z, x.w});
}
__device__ __forceinline__ bf16x4 frag_a16(const bf16* p, int ld, int lane) {
    return *reinterpret_cast<const bf16x4*>(p + (lane & 15) * ld + 4 * (lane >> 4));
}
// 16x16x16 B operand of a 16x16 block at `p` (row-major): lane 16g+n holds
// X[4g..4g+3][n]
__device__ __forceinline__ bf16x4 frag_b16(const float* p, int ld, int lane) {
    const float* q = p + 4 * (lane >> 4) * ld + (lane & 15);
    return to_bf4(f32x4{q[0], q[ld], q[2 * ld], q[3 * ld]});
}
// the same 4 x 16 slice of a row-major bf16 block with one transposing read
// (lane j of each 16-lane group addresses row 4g + j/4, columns 4(j%4)..+3)
__device__ __forceinline__ bf16x4 tr_b16(const bf16* p, int ld, int lane) {
    const int g = lane >> 4, j = lane & 15;
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(p + (4 * g + (j >> 2)) * ld + 4 * (j & 3)));
    return __builtin_bit_cast(bf16x4, v);
}
// an accumulator tile used as the next 16x16x16 B operand (same layout)
__device__ __forceinline__ bf16x4 acc_b16(f32x4 v) { return to_bf4(v); }
// store a 16x16 accumulator tile into a row-major fp32 block
__device__ __forceinline__ void store_blk(float* p, int ld, int lane, f32x4 v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) p[(4 * (lane >> 4) + e) * ld + (lane & 15)] = v[e];
}
// the same wave reads back what it wrote to LDS
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0) only: leave vector-memory loads in flight
    __builtin_amdgcn_wave_barrier();
}
// 16x16x32 A operand of rows of T (fp32, row-major): lane 16g+m holds
// T[m][k0+8g..k0+8g+7]
__device__ __forceinline__ M::frag frag_t(const float* trow, int k0, int lane) {
    const int c0 = k0 + 8 * (lane >> 4);
    const float4 x0 = *reinterpret_cast<const float4*>(trow + c0);
    const float4 x1 = *reinterpret_cast<const float4*>(trow + c0 + 4);
    const u32x4 w{pack_bf16x2(x0.x, x0.y), pack_bf16x2(x0.z, x0.w), pack_bf16x2(x1.x, x1.y),
                  pack_bf16x2(x1.z, x1.w)};
    return __builtin_bit_cast(bf16x8, w);
}

// Inclusive prefix sum over the 64 lanes with DPP moves (row shifts inside
// each 16-lane row, then the row-15 and row-31 broadcasts across rows): no
// LDS traffic, unlike a shuffle-based scan.  Lanes whose source is outside
// the row, or whose row is masked off, add 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float add_dpp(float v) {
    return v + __int_as_float(
                   __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}
__device__ __forceinline__ float wave_scan_dpp(float x) {
    x = add_dpp<0x111, 0xf>(x);   // row_shr:1
    x = add_dpp<0x112, 0xf>(x);   // row_shr:2
    x = add_dpp<0x114, 0xf>(x);   // row_shr:4
    x = add_dpp<0x118, 0xf>(x);   // row_shr:8
    x = add_dpp<0x142, 0xa>(x);   // row_bcast:15 into rows 1 and 3
    x = add_dpp<0x143, 0xc>(x);   // row_bcast:31 into rows 2 and 3
    return x;
}

// Chunk inputs held in registers between their load and their LDS store.
struct Stage {
    u32x4 k[2], q[2];
    u32x2 v;
    float g, b;
};

struct Ctx {
    const bf16 *q, *k, *v;
    const float *beta, *g;
    int64_t H, h, t0, len;
    int v0, nch, tid, lane, wave;
    float scale;
    char* smem;

    __device__ __forceinline__ bf16* sK(int c) const {
        return reinterpret_cast<bf16*>(smem + o_K + SZ_KQ * (c % 3));
    }
    __device__ __forceinline__ bf16* sQ() const { return reinterpret_cast<bf16*>(smem + o_Q); }
    __device__ __forceinline__ bf16* sV() const { return reinterpret_cast<bf16*>(smem + o_V); }
    // off-diagonal blocks of A: row i (16 <= i < 64) at row i - 16, column j < 48
    __device__ __forceinline__ bf16* sA() const { return reinterpret_cast<bf16*>(smem + o_A); }
    __device__ __forceinline__ float* sN() const { return reinterpret_cast<float*>(smem + o_N); }
    __device__ __forceinline__ float* sT(int c) const {
        return reinterpret_cast<float*>(smem + o_T + SZ_T * (c & 1));
    }
    __device__ __forceinline__ bf16* shT() const { return reinterpret_cast<bf16*>(smem + o_hT); }
    __device__ __forceinline__ bf16* sR() const { return reinterpret_cast<bf16*>(smem + o_R); }
    __device__ __forceinline__ bf16* sVn() const { return reinterpret_cast<bf16*>(smem + o_Vn); }
    __device__ __forceinline__ bf16* sVt() const { return reinterpret_cast<bf16*>(smem + o_Vt); }
    __device__ __forceinline__ float* gate(int c, int which) const {
        return reinterpret_cast<float*>(smem + o_Gt) + ((c % 3) * NGA + which) * C;
    }
    __device__ __forceinline__ bool valid(int c) const { return c >= 0 && c < nch; }
    __device__ __forceinline__ int rows(int c) const {
        return (int)min((int64_t)C, len - (int64_t)c * C);
    }

    // ---- loads into registers.  Chunk indices are clamped into [0, nch) so
    // that every wave issues the same loads every iteration: the compiler can
    // then count them and wait only for the ones a store needs, not for the
    // loads issued for later iterations.  (Loads of clamped indices land in
    // slots no live chunk uses.)
    __device__ __forceinline__ int clampc(int c) const { return min(max(c, 0), nch - 1); }
    // byte offset of row r (clamped to the chunk's last row) from the chunk's
    // first row, plus a column offset; rows are H*D elements apart
    __device__ __forceinline__ uint32_t roff(int c, int r, int D, int colbytes) const {
        return (uint32_t)min(r, rows(c) - 1) * (uint32_t)(H * D * 2) + (uint32_t)colbytes;
    }
    template <typename P>
    __device__ __forceinline__ const char* chunk_row0(const P* base, int c, int D) const {
        return reinterpret_cast<const char*>(base + ((t0 + (int64_t)c * C) * H + h) * D);
    }
    // everything iteration j stores: K_{j+2} and gates_{j+2}, V_{j+1}, Q_{j+1}
    // (the gates only in the wave that stores them: a load whose register is
    // never read would make the compiler wait for it before reusing the register)
    template <bool GATES>
    __device__ __forceinline__ void load_for(Stage& s, int j) const {
        const int cv = clampc(j + 1), ck = clampc(j + 2);
        const char* vb = chunk_row0(v, cv, V) + v0 * 2;
        const char* kb = chunk_row0(k, ck, K);
        const char* qb = chunk_row0(q, cv, K);
        s.v = *reinterpret_cast<const u32x2*>(vb + roff(cv, tid >> 3, V, (tid & 7) * 8));
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int i = tid + NT * p;
            s.k[p] = *reinterpret_cast<const u32x4*>(kb + roff(ck, i >> 4, K, (i & 15) * 16));
            s.q[p] = *reinterpret_cast<const u32x4*>(qb + roff(cv, i >> 4, K, (i & 15) * 16));
        }
        if constexpr (GATES) {
            // rows past a ragged end re-read the last row; store_gates zeroes them
            const uint32_t go = (uint32_t)min(lane, rows(ck) - 1) * (uint32_t)(H * 4);
            s.g = *reinterpret_cast<const float*>(chunk_row0(g, ck, 1) + go);
            s.b = *reinterpret_cast<const float*>(chunk_row0(beta, ck, 1) + go);
        }
    }

    // ---- LDS stores of staged inputs
    __device__ __forceinline__ void store_k(const Stage& s, int c) const {
        bf16* d = sK(c);
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int i = tid + NT * p;
            *reinterpret_cast<u32x4*>(d + (i >> 4) * LDK + (i & 15) * 8) = s.k[p];
        }
    }
    __device__ __forceinline__ void store_q(const Stage& s) const {
        bf16* d = sQ();
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int i = tid + NT * p;
            *reinterpret_cast<u32x4*>(d + (i >> 4) * LDK + (i & 15) * 8) = s.q[p];
        }
    }
    __device__ __forceinline__ void store_v(const Stage& s) const {
        *reinterpret_cast<u32x2*>(sV() + (tid >> 3) * LDVS + (tid & 7) * 4) = s.v;
    }
    // cumulative log2 gate and the per-row factors derived from it (one wave,
    // lane = row; rows past the chunk end carry g = 0 and beta = 0)
    __device__ __forceinline__ void store_gates(const Stage& s, int c) const {
        const bool in = lane < rows(c);
        const float G = wave_scan_dpp(in ? s.g * LOG2E : 0.f);
        const float bt = in ? s.b : 0.f;
        const float Gc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(G), C - 1));
        const float gam = exp2_hw(G);
        gate(c, G_LOG)[lane] = G;
        gate(c, G_BETA)[lane] = bt;
        gate(c, G_OUT)[lane] = scale * gam;
        gate(c, G_TAIL)[lane] = exp2_hw(fminf(Gc - G, 0.f));
        gate(c, G_GAM)[lane] = gam;
        gate(c, G_END)[lane] = exp2_hw(Gc);
        // G at the first token of each 16-token block
        float Gs[4];
#pragma unroll
        for (int I = 0; I < 4; ++I)
            Gs[I] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(G), 16 * I));
        const int bl = lane >> 4;
        const float Gb = bl == 0 ? Gs[0] : bl == 1 ? Gs[1] : bl == 2 ? Gs[2] : Gs[3];
        gate(c, G_ROW)[lane] = exp2_hw(fminf(G - Gb, 0.f));
#pragma unroll
        for (int I = 1; I < 4; ++I)
            gate(c, G_COL + I - 1)[lane] = exp2_hw(fminf(Gs[I] - G, 0.f));
    }
};

// ---------------------------------------------------------------- intra parts
// S^T tile (J, I) = X_J Y_I^T over the full key dimension (X, Y row blocks of
// K or Q): lane 16g+n holds S[16I + n][16J + 4g + e]
__device__ __forceinline__ f32x4 kk_t(const bf16* a_rows, const bf16* b_rows, int lane) {
    f32x4 acc = zero4();
    const bf16* ar = a_rows + (lane & 15) * LDK;
    const bf16* br = b_rows + (lane & 15) * LDK;
    M::frag fa[K / 32], fb[K / 32];
#pragma unroll
    for (int s = 0; s < K / 32; ++s) {
        fa[s] = M::load(ar + 32 * s, lane);
        fb[s] = M::load(br + 32 * s, lane);
    }
#pragma unroll
    for (int s = 0; s < K / 32; ++s) acc = M::mma(fa[s], fb[s], acc);
    return acc;
}

// off-diagonal block (I, J), I > J, of A: beta_i 2^{G_i - G_j} k_i.k_j -> sA (bf16)
__device__ __forceinline__ void a_offdiag(const Ctx& x, int c, int I, int J) {
    const bf16* kk = x.sK(c);
    const int i = 16 * I + (x.lane & 15), j0 = 16 * J + 4 * (x.lane >> 4);
    const float bi = x.gate(c, G_BETA)[i], rw = x.gate(c, G_ROW)[i];
    const float4 cj = *reinterpret_cast<const float4*>(x.gate(c, G_COL + I - 1) + j0);
    const f32x4 s = kk_t(kk + 16 * J * LDK, kk + 16 * I * LDK, x.lane);
    const float ri = bi * rw;
    store4(x.sA() + (i - 16) * LDA + j0,
           f32x4{ri * cj.x * s[0], ri * cj.y * s[1], ri * cj.z * s[2], ri * cj.w * s[3]});
}

// diagonal block b of A (strictly lower), transposed into sN[b]: sN[b][r][m] = A[16b+m][16b+r]
__device__ __forceinline__ void a_diag(const Ctx& x, int c, int b) {
    const bf16* kb = x.sK(c) + 16 * b * LDK + (x.lane & 15) * LDK;
    M::frag f[K / 32];
#pragma unroll
    for (int k0 = 0; k0 < K / 32; ++k0) f[k0] = M::load(kb + 32 * k0, x.lane);
    // lane 16g+n: S[16b + 4g + e][16b + n], i.e. A row m = 4g+e, column r = n
    const float* G = x.gate(c, G_LOG) + 16 * b;
    const float* B = x.gate(c, G_BETA) + 16 * b;
    const int r = x.lane & 15, m0 = 4 * (x.lane >> 4);
    const float gr = G[r];
    const float4 gm4 = *reinterpret_cast<const float4*>(G + m0);
    const float4 bm4 = *reinterpret_cast<const float4*>(B + m0);
    f32x4 s = zero4();
#pragma unroll
    for (int k0 = 0; k0 < K / 32; ++k0) s = M::mma(f[k0], f[k0], s);
    const float gm[4] = {gm4.x, gm4.y, gm4.z, gm4.w}, bm[4] = {bm4.x, bm4.y, bm4.z, bm4.w};
    float4 o;
    float* op = &o.x;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        op[e] = r < m0 + e ? bm[e] * exp2_hw(fminf(gm[e] - gr, 0.f)) * s[e] : 0.f;
    *reinterpret_cast<float4*>(x.sN() + b * NBS + r * LDN + m0) = o;
}

// forward substitution of the four 16x16 diagonal blocks of I + A (one wave;
// lane 16b+c computes column c of (I + N_b)^{-1}), written into the diagonal
// blocks of T.  Column sweep: after step r, x_r is final and later rows have
// subtracted N[m][r] x_r.  Rows of N^T are read LA steps ahead; the compiler
// barrier keeps it from hoisting every read (which would take ~240 VGPRs).
__device__ __forceinline__ void diag_inverse(const Ctx& x, int c) {
    constexpr int LA = 3;
    const int b = x.lane >> 4, col = x.lane & 15;
    const float* nb = x.sN() + b * NBS;
    float xv[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) xv[m] = (m == col) ? 1.f : 0.f;
    float4 buf[LA + 1][4];
#pragma unroll
    for (int r = 0; r < LA; ++r)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            buf[r][q4] = *reinterpret_cast<const float4*>(nb + r * LDN + 4 * q4);
#pragma unroll
    for (int r = 0; r < 15; ++r) {
        if (r + LA < 15) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                buf[(r + LA) % (LA + 1)][q4] =
                    *reinterpret_cast<const float4*>(nb + (r + LA) * LDN + 4 * q4);
        }
        const float* cl = reinterpret_cast<const float*>(buf[r % (LA + 1)]);
#pragma unroll
        for (int m = r + 1; m < 16; ++m) xv[m] -= cl[m] * xv[r];
        __asm__ volatile("" ::: "memory");
    }
    float* tb = x.sT(c) + 16 * b * LDT + 16 * b + col;
#pragma unroll
    for (int m = 0; m < 16; ++m) tb[m * LDT] = xv[m];
}

// Off-diagonal blocks of T from the diagonal ones (bf16 MFMA, fp32 results):
// wave 0 writes T10, T20, T21; wave 1 writes T32, T30, T31 (and recomputes the
// T10 it needs in registers).
__device__ __forceinline__ void compose(const Ctx& x, int c, int which) {
    float* T = x.sT(c);
    const bf16* A = x.sA();
    const int l = x.lane;
    auto Tb = [&](int I, int J) { return T + 16 * I * LDT + 16 * J; };
    auto Ab = [&](int I, int J) { return A + (16 * I - 16) * LDA + 16 * J; };
    const bf16x4 t00b = frag_b16(Tb(0, 0), LDT, l), t11b = frag_b16(Tb(1, 1), LDT, l);
    // T10 = -T11 (A10 T00)
    const f32x4 x10 = mma16(frag_a16(Ab(1, 0), LDA, l), t00b, zero4());
    const f32x4 t10 = mma16(frag_a16(Tb(1, 1), LDT, l), acc_b16(-x10), zero4());
    const bf16x4 t10b = acc_b16(t10);
    const bf16x4 a21 = frag_a16(Ab(2, 1), LDA, l);
    // P20 = A20 T00 + A21 T10, P21 = A21 T11
    f32x4 p20 = mma16(frag_a16(Ab(2, 0), LDA, l), t00b, zero4());
    p20 = mma16(a21, t10b, p20);
    const f32x4 p21 = mma16(a21, t11b, zero4());
    if (which == 0) {
        store_blk(Tb(1, 0), LDT, l, t10);
        const bf16x4 t22a = frag_a16(Tb(2, 2), LDT, l);
        store_blk(Tb(2, 0), LDT, l, mma16(t22a, acc_b16(-p20), zero4()));
        store_blk(Tb(2, 1), LDT, l, mma16(t22a, acc_b16(-p21), zero4()));
    } else {
        // T32 = -T33 (A32 T22)
        const f32x4 x32 = mma16(frag_a16(Ab(3, 2), LDA, l), frag_b16(Tb(2, 2), LDT, l), zero4());
        const bf16x4 t33a = frag_a16(Tb(3, 3), LDT, l);
        const f32x4 t32 = mma16(t33a, acc_b16(-x32), zero4());
        store_blk(Tb(3, 2), LDT, l, t32);
        const bf16x4 a31 = frag_a16(Ab(3, 1), LDA, l);
        f32x4 p30 = mma16(frag_a16(Ab(3, 0), LDA, l), t00b, zero4());
        p30 = mma16(a31, t10b, p30);
        const f32x4 p31 = mma16(a31, t11b, zero4());
        wave_lds_sync();
        const bf16x4 t32a = frag_a16(Tb(3, 2), LDT, l);
        // T3J = -(T32 P2J + T33 P3J)
        f32x4 t30 = mma16(t32a, acc_b16(-p20), zero4());
        t30 = mma16(t33a, acc_b16(-p30), t30);
        f32x4 t31 = mma16(t32a, acc_b16(-p21), zero4());
        t31 = mma16(t33a, acc_b16(-p31), t31);
        store_blk(Tb(3, 0), LDT, l, t30);
        store_blk(Tb(3, 1), LDT, l, t31);
    }
}

// ---------------------------------------------------------------- the kernel
// off-diagonal K K^T blocks (I, J) of waves 5, 6, 7 (two each) in the second phase
__constant__ int AO_I[6] = {3, 3, 3, 2, 2, 1};
__constant__ int AO_J[6] = {0, 1, 2, 0, 1, 0};

// Everything a wave of role R (0: V waves, 1: O waves, 2: H waves) does; the
// role is a compile-time constant so that each loop holds only its role's
// values in registers, and the wave index inside the role is a runtime value
// so that the kernel's code (three loops) stays well inside the instruction
// cache.  Every wave executes the same barriers in the same order.
template <int R, int SUB>
__device__ __forceinline__ void run_role(Ctx& x, const FusedLaunch& a, int64_t n) {
    constexpr bool VW = R == 0, OW = R == 1, HW = R == 2;
    constexpr bool GW = VW && SUB == 0;   // the wave that computes the gate arrays
    // wave index: a compile-time constant for the V and O waves (whose work
    // differs by block), a runtime value for the four H waves
    const int W = HW ? x.wave : (VW ? SUB : 2 + SUB);
    const int lane = x.lane;
    f32x4 hacc[2][CT];   // H waves: h rows 32p.., fp32
    if constexpr (HW) {
        const int p = W - 4;
        const float* h0 = a.h0 ? a.h0 + (n * a.H + x.h) * (int64_t)(K * V) : nullptr;
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    hacc[r][ct][e] = h0 ? h0[(16 * (2 * p + r) + acc_row(lane, e)) * V + x.v0 +
                                             16 * ct + acc_col(lane)]
                                        : 0.f;
                store_acc_t(x.shT() + 16 * ct * LDH + 16 * (2 * p + r), LDH, lane, hacc[r][ct]);
            }
    }

    Stage st[PD];
    if (x.nch > 0) {
#pragma unroll
    for (int s = 0; s < PD; ++s) x.load_for<GW>(st[s], s - 2);

    auto iteration = [&](Stage& s, int j) __attribute__((always_inline)) {
        const int c1 = j + 1, c2 = j + 2;
        const bool scan = j >= 0, in1 = x.valid(c1);
        f32x4 oacc[CT][2];   // O waves: O^T of their token blocks
        f32x4 sq[2][4];      // O waves: off-diagonal causal blocks (J, I), J < I, fp32
        f32x4 sqd[2] = {zero4(), zero4()};   // O waves: diagonal causal blocks
        bf16x4 aq[2][4];     // O waves: causal Q K^T blocks (J, I), 16x16x16 B operands
        // wave 2 owns token blocks 0 and 3, wave 3 blocks 1 and 2: both then
        // have five causal Q K^T blocks
        constexpr int ib0 = SUB == 1 ? 1 : 0, ib1 = SUB == 1 ? 2 : 3;
        // ================= P1
        // Staged inputs are stored unconditionally (clamped duplicates for
        // chunks past the end land in slots no live chunk uses), so that no
        // staged register is left with a load in flight on some path.
        x.store_k(s, c2);
        if constexpr (VW) {
            if (scan) {
                // R = diag(beta) (V - diag(gamma) K h) for token rows 32m..32m+31
                constexpr int m = SUB;
                const bf16* kk = x.sK(j);
                const float* bt = x.gate(j, G_BETA);
                const float* gm = x.gate(j, G_GAM);
                float4 b4[2], g4[2];
                bf16x4 vv[2][CT];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int r0 = 32 * m + 16 * t;
                    b4[t] = *reinterpret_cast<const float4*>(bt + r0 + 4 * (lane >> 4));
                    g4[t] = *reinterpret_cast<const float4*>(gm + r0 + 4 * (lane >> 4));
                    // V rows r0+4g+e, column 16ct+n: the accumulator's layout
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct)
                        vv[t][ct] = tr_b16(x.sV() + r0 * LDVS + 16 * ct, LDVS, lane);
                }
                f32x4 acc[2][CT];
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) acc[t][ct] = zero4();
#pragma unroll
                for (int sg = 0; sg < K / 32; ++sg) {
                    const M::frag a0 = M::load(kk + (32 * m + (lane & 15)) * LDK + 32 * sg, lane);
                    const M::frag a1 =
                        M::load(kk + (32 * m + 16 + (lane & 15)) * LDK + 32 * sg, lane);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) {
                        const M::frag bh =
                            M::load(x.shT() + (16 * ct + (lane & 15)) * LDH + 32 * sg, lane);
                        acc[0][ct] = M::mma(a0, bh, acc[0][ct]);
                        acc[1][ct] = M::mma(a1, bh, acc[1][ct]);
                    }
                }
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int r0 = 32 * m + 16 * t;
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) {
                        const bf16x4 v4 = vv[t][ct];
                        const f32x4 r{b4[t].x * ((float)v4[0] - g4[t].x * acc[t][ct][0]),
                                      b4[t].y * ((float)v4[1] - g4[t].y * acc[t][ct][1]),
                                      b4[t].z * ((float)v4[2] - g4[t].z * acc[t][ct][2]),
                                      b4[t].w * ((float)v4[3] - g4[t].w * acc[t][ct][3])};
                        store_acc_t(x.sR() + 16 * ct * LDVN + r0, LDVN, lane, r);
                    }
                }
            }
        }
        if constexpr (OW) {
            if (scan) {
                // O^T = h^T Q^T for the two token blocks, and the
                // off-diagonal causal blocks S^T(J, I) = K_J Q_I^T, J < I
                const bf16* kk = x.sK(j);
                const float* og = x.gate(j, G_OUT);
                const float s0 = og[16 * ib0 + (lane & 15)], s1 = og[16 * ib1 + (lane & 15)];
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) oacc[ct][0] = oacc[ct][1] = zero4();
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int J = 0; J < 4; ++J) sq[t][J] = zero4();
#pragma unroll
                for (int sg = 0; sg < K / 32; ++sg) {
                    const M::frag b0 =
                        M::load(x.sQ() + (16 * ib0 + (lane & 15)) * LDK + 32 * sg, lane);
                    const M::frag b1 =
                        M::load(x.sQ() + (16 * ib1 + (lane & 15)) * LDK + 32 * sg, lane);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) {
                        const M::frag ah =
                            M::load(x.shT() + (16 * ct + (lane & 15)) * LDH + 32 * sg, lane);
                        oacc[ct][0] = M::mma(ah, b0, oacc[ct][0]);
                        oacc[ct][1] = M::mma(ah, b1, oacc[ct][1]);
                    }
#pragma unroll
                    for (int J = 0; J < 3; ++J) {
                        if (J >= ib0 && J >= ib1) continue;
                        const M::frag kf =
                            M::load(kk + (16 * J + (lane & 15)) * LDK + 32 * sg, lane);
                        if (J < ib0) sq[0][J] = M::mma(kf, b0, sq[0][J]);
                        if (J < ib1) sq[1][J] = M::mma(kf, b1, sq[1][J]);
                    }
                }
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    oacc[ct][0] *= s0;
                    oacc[ct][1] *= s1;
                }
            }
        }
        if constexpr (HW) {
            if (scan) {
                const float dec = x.gate(j, G_END)[0];
#pragma unroll
                for (int r = 0; r < 2; ++r)
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) hacc[r][ct] *= dec;
            }
            if (in1) a_diag(x, c1, W - 4);
        }
        __syncthreads();
        // ================= P2
        x.store_v(s);
        if constexpr (VW) {
            if (scan) {
                // V_new = T R for token rows 32m..32m+31 (T is zero above the
                // diagonal, so k-steps past the rows' own block add nothing)
                constexpr int m = SUB;
                const float* T = x.sT(j);
                const float* tail = x.gate(j, G_TAIL);
                float4 f4[2];
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    f4[t] = *reinterpret_cast<const float4*>(tail + 32 * m + 16 * t + 4 * (lane >> 4));
                f32x4 vn[2][CT];
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) vn[t][ct] = zero4();
#pragma unroll
                for (int sg = 0; sg < 2; ++sg) {
                    if (sg > m) break;
                    M::frag bt[CT];
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct)
                        bt[ct] = M::load(x.sR() + (16 * ct + (lane & 15)) * LDVN + 32 * sg, lane);
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const M::frag at =
                            frag_t(T + (32 * m + 16 * t + (lane & 15)) * LDT, 32 * sg, lane);
#pragma unroll
                        for (int ct = 0; ct < CT; ++ct) vn[t][ct] = M::mma(at, bt[ct], vn[t][ct]);
                    }
                }
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int r0 = 32 * m + 16 * t;
                    const float4 f = f4[t];
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) {
                        const f32x4 v = vn[t][ct];
                        store_acc_t(x.sVn() + 16 * ct * LDVN + r0, LDVN, lane, v);
                        store_acc_t(x.sVt() + 16 * ct * LDVN + r0, LDVN, lane,
                                    f32x4{f.x * v[0], f.y * v[1], f.z * v[2], f.w * v[3]});
                    }
                }
            }
        }
        if constexpr (OW) {
            if (scan) {
                // the diagonal causal blocks S^T(I, I) = K_I Q_I^T
                const bf16* kk = x.sK(j);
#pragma unroll
                for (int sg = 0; sg < K / 32; ++sg) {
                    const M::frag b0 =
                        M::load(x.sQ() + (16 * ib0 + (lane & 15)) * LDK + 32 * sg, lane);
                    const M::frag b1 =
                        M::load(x.sQ() + (16 * ib1 + (lane & 15)) * LDK + 32 * sg, lane);
                    const M::frag k0 =
                        M::load(kk + (16 * ib0 + (lane & 15)) * LDK + 32 * sg, lane);
                    const M::frag k1 =
                        M::load(kk + (16 * ib1 + (lane & 15)) * LDK + 32 * sg, lane);
                    sqd[0] = M::mma(k0, b0, sqd[0]);
                    sqd[1] = M::mma(k1, b1, sqd[1]);
                }
                // every gate value the masks need, read before any is used
                const float* G = x.gate(j, G_LOG);
                const float* ROW = x.gate(j, G_ROW);
                const int g4 = 4 * (lane >> 4);
                float gi[2], si[2];
                float4 gd[2], cj[2][3];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int I = t ? ib1 : ib0, i = 16 * I + (lane & 15);
                    gi[t] = G[i];
                    si[t] = x.scale * ROW[i];
                    gd[t] = *reinterpret_cast<const float4*>(G + 16 * I + g4);
#pragma unroll
                    for (int J = 0; J < I; ++J)
                        cj[t][J] =
                            *reinterpret_cast<const float4*>(x.gate(j, G_COL + I - 1) + 16 * J + g4);
                }
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int I = t ? ib1 : ib0, i = 16 * I + (lane & 15);
                    // lane 16g+n of tile (J, I) holds S[i = 16I+n][j = 16J+4g+e];
                    // off-diagonal blocks use the factored decay, the diagonal
                    // block the direct one and the causal mask
#pragma unroll
                    for (int J = 0; J < I; ++J)
                        aq[t][J] = to_bf4(f32x4{si[t] * cj[t][J].x * sq[t][J][0],
                                                si[t] * cj[t][J].y * sq[t][J][1],
                                                si[t] * cj[t][J].z * sq[t][J][2],
                                                si[t] * cj[t][J].w * sq[t][J][3]});
                    const float gdv[4] = {gd[t].x, gd[t].y, gd[t].z, gd[t].w};
                    f32x4 av;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int jj = 16 * I + g4 + e;
                        av[e] = jj <= i ? x.scale * exp2_hw(fminf(gi[t] - gdv[e], 0.f)) * sqd[t][e]
                                        : 0.f;
                    }
                    aq[t][I] = to_bf4(av);
                }
            }
        }
        if constexpr (HW) {
            if (in1) {
                if (W == 4) {
                    // on the SIMD it shares with wave 0, whose second phase is light
                    diag_inverse(x, c1);
                } else {
                    // waves 5, 6, 7 take blocks (3,0) (3,1) | (3,2) (2,0) | (2,1) (1,0)
                    const int q = W - 5;
                    a_offdiag(x, c1, AO_I[2 * q], AO_J[2 * q]);
                    a_offdiag(x, c1, AO_I[2 * q + 1], AO_J[2 * q + 1]);
                }
            }
        }
        __syncthreads();
        // ================= P3
        x.store_q(s);
        // gates of chunk j+2 (first read in the next iteration's first phase)
        if constexpr (GW) x.store_gates(s, c2);
        x.load_for<GW>(s, j + PD);
        if constexpr (VW) {
            if (in1) compose(x, c1, SUB);
        }
        if constexpr (OW) {
            if (scan) {
                // + V_new^T Aqk^T over the causal blocks J <= I (16x16x16:
                // lane 16g+m reads V_new^T[16ct+m][16J+4g..+3])
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int I = t ? ib1 : ib0;
#pragma unroll
                    for (int J = 0; J < 4; ++J) {
                        if (J > I) continue;
#pragma unroll
                        for (int ct = 0; ct < CT; ++ct)
                            oacc[ct][t] = mma16(
                                frag_a16(x.sVn() + 16 * ct * LDVN + 16 * J, LDVN, lane), aq[t][J],
                                oacc[ct][t]);
                    }
                }
                const int ntok = x.rows(j);
                const int64_t tt0 = x.t0 + (int64_t)j * C;
                bf16* o = static_cast<bf16*>(a.o);
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int tk = 16 * (t ? ib1 : ib0) + acc_col(lane);
                    if (tk < ntok) {
#pragma unroll
                        for (int ct = 0; ct < CT; ++ct)
                            store4(o + ((tt0 + tk) * a.H + x.h) * V + x.v0 + 16 * ct +
                                       4 * (lane >> 4),
                                   oacc[ct][t]);
                    }
                }
            }
        }
        if constexpr (HW) {
            if (scan) {
                const int p = W - 4;
                const bf16* kk = x.sK(j);
#pragma unroll
                for (int sg = 0; sg < C / 32; ++sg) {
                    const M::frag a0 = M::load_t(kk + 32 * sg * LDK + 32 * p, LDK, lane);
                    const M::frag a1 = M::load_t(kk + 32 * sg * LDK + 32 * p + 16, LDK, lane);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) {
                        const M::frag bv =
                            M::load(x.sVt() + (16 * ct + (lane & 15)) * LDVN + 32 * sg, lane);
                        hacc[0][ct] = M::mma(a0, bv, hacc[0][ct]);
                        hacc[1][ct] = M::mma(a1, bv, hacc[1][ct]);
                    }
                }
#pragma unroll
                for (int r = 0; r < 2; ++r)
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct)
                        store_acc_t(x.shT() + 16 * ct * LDH + 16 * (2 * p + r), LDH, lane,
                                    hacc[r][ct]);
            }
        }
        __syncthreads();
    };

    int j = -2;
    for (; j + PD <= x.nch; j += PD) {
        iteration(st[0], j);
        iteration(st[1], j + 1);
    }
    if (j < x.nch) iteration(st[0], j);
    }

    if constexpr (HW) {
        if (a.ht) {
            const int p = W - 4;
            float* ht = a.ht + (n * a.H + x.h) * (int64_t)(K * V);
#pragma unroll
            for (int r = 0; r < 2; ++r)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        ht[(16 * (2 * p + r) + acc_row(lane, e)) * V + x.v0 + 16 * ct +
                           acc_col(lane)] = hacc[r][ct][e];
        }
    }
}

__global__ __launch_bounds__(NT) void fused_kernel(FusedLaunch a) {
    __shared__ __attribute__((aligned(16))) char smem[BYTES];
    const int64_t bid = blockIdx.x;
    const int vt = (int)((bid >> 3) % NVT);
    const int64_t chain = (bid & 7) + 8 * ((bid >> 3) / NVT);
    if (chain >= a.N * a.H) return;

    Ctx x;
    x.q = static_cast<const bf16*>(a.q);
    x.k = static_cast<const bf16*>(a.k);
    x.v = static_cast<const bf16*>(a.v);
    x.beta = a.beta;
    x.g = a.g;
    x.H = a.H;
    const int64_t n = chain / a.H;
    x.h = chain - n * a.H;
    x.v0 = vt * VT;
    x.tid = threadIdx.x;
    x.lane = threadIdx.x & 63;
    x.wave = wave_id();
    x.scale = a.scale;
    x.smem = smem;
    if (a.seqs) {
        const int4 s = a.seqs[n];
        x.t0 = s.x;
        x.len = s.y;
    } else {
        x.t0 = n * a.T;
        x.len = a.T;
    }
    x.nch = (int)((x.len + C - 1) / C);

    // zero both T slots: their upper blocks are read as zeros
    for (int i = x.tid; i < 2 * C * LDT; i += NT) x.sT(0)[i] = 0.f;

    switch (x.wave) {
        case 0: run_role<0, 0>(x, a, n); break;
        case 1: run_role<0, 1>(x, a, n); break;
        case 2: run_role<1, 0>(x, a, n); break;
        case 3: run_role<1, 1>(x, a, n); break;
        default: run_role<2, 0>(x, a, n); break;
    }
}

}  // namespace fz

bool fused_supported(const FusedLaunch& a) {
    return a.bf16 && !a.per_key && a.K == fz::K && a.V == fz::V && a.C == fz::C;
}

hipError_t launch_fused(const FusedLaunch& a) {
    if (!fused_supported(a)) return hipErrorInvalidValue;
    const int64_t chains = a.N * a.H;
    const int64_t nblk = ((chains + 7) / 8) * 8 * fz::NVT;
    hipLaunchKernelGGL(fz::fused_kernel, dim3((unsigned)nblk), dim3(fz::NT), 0, a.stream, a);
    return hipGetLastError();
}

}  // namespace gdn
