// Body of the fused chunked forward (k_fused.hip), compiled once per head
// size: it is included inside a namespace that defines the constants K (key
// head size) and V (value head size), each 64 or 128.  No include guard on
// purpose.

constexpr int C = 64, VT = 32, NVT = V / VT;
static_assert((K == 64 || K == 128) && (V == 64 || V == 128), "head sizes");
constexpr int NT = 512;
// K-dependent counts: 32-channel steps of the K h / K K^T products, 16-row
// state tiles, 16-byte groups per K/Q row (= 1 KB loads per K/Q chunk)
constexpr int NKK = K / 32, NST = K / 16, GPR = K / 8;

// ---------------------------------------------------------------- LDS layout
// K, Q: 64 rows of 2K bytes; the 16-byte group holding columns 8q..8q+7 of
// row r sits at position q ^ (2r mod 16) for K = 128 and q ^ (r & 6) for
// K = 64, whose 128-byte rows cover half the banks, so rows r and r + 1 sit
// in different halves and the permutation only has to separate rows of equal
// parity (measured: 36 % of LDS cycles in bank conflicts with q ^ (2r mod 8),
// 22 % with this one, as at K = 128).  V (the 32-column slice): 64 rows of
// 64 bytes, group q of row r at q ^ 2((r/4)%2).  Pitches and permutations are
// the ones measured free of LDS bank conflicts on gfx950 for the reads made
// here: 16-byte row fragments need rows an odd multiple of 32 bytes apart
// (or this permutation of 2K-byte rows, which also serves the transposing
// K^T reads), 8-byte row reads an odd multiple of 8 bytes.
constexpr int SZ_KQ = C * 2 * K;
constexpr int SZ_V = C * VT * 2;
constexpr int SZ_RAW = 2 * C * 4;    // g and beta as loaded
constexpr int NGA = 10;              // gate arrays per chunk
constexpr int SZ_G = NGA * C * 4;
constexpr int SZ_AQ = 6 * 64 * 16;   // six causal 16x16x32 fragments of Aqk
constexpr int LDTT = 80;             // bf16 per row of T^T (160 bytes)
constexpr int SZ_TT = C * LDTT * 2;
constexpr int LDAB = 20;             // bf16 per row of an off-diagonal A block (40 bytes)
constexpr int SZ_AB = 16 * LDAB * 2;
constexpr int SZ_A = 6 * SZ_AB;
constexpr int LDD = 24;              // fp32 per row of a diagonal A block (96 bytes)
constexpr int SZ_DB = 16 * LDD * 4;
constexpr int LDDT = 20;             // bf16 per row of a 16x16 block of D^T (40 bytes)
constexpr int SZ_DT = 16 * LDDT * 2;

constexpr int o_K = 0;                       // 3 slots
constexpr int o_Q = o_K + 3 * SZ_KQ;         // 3 slots
constexpr int o_V = o_Q + 3 * SZ_KQ;         // 3 slots
constexpr int o_RAW = o_V + 3 * SZ_V;        // 2 slots
constexpr int o_G = o_RAW + 2 * SZ_RAW;      // 3 slots
constexpr int o_AQ = o_G + 3 * SZ_G;         // 2 slots
constexpr int o_TT = o_AQ + 2 * SZ_AQ;
constexpr int o_A = o_TT + SZ_TT;            // 2 slots
constexpr int o_D = o_A + 2 * SZ_A;
constexpr int o_DT = o_D + 4 * SZ_DB;
constexpr int o_F = o_DT + 4 * SZ_DT;        // signal words
constexpr int BYTES = o_F + 64;
// the q/k L2-normalising instantiation only: per product wave, squared
// norms of the chunk's tokens: the key wave's |k|^2 (read by the query waves
// too, once signalled) and each query set's |q|^2 (in [64, 128))
constexpr int SZ_NRM = 128 * 4;
constexpr int o_NRM = BYTES;
constexpr int BYTES_L2 = o_NRM + 4 * SZ_NRM;
static_assert(BYTES_L2 <= 160 * 1024, "LDS budget of one workgroup");
static_assert(o_V % 16 == 0 && o_RAW % 16 == 0 && o_G % 16 == 0 && o_AQ % 16 == 0 && o_TT % 16 == 0 &&
                  o_A % 16 == 0 && o_D % 16 == 0 && o_DT % 16 == 0 && o_F % 16 == 0 && o_NRM % 16 == 0,
              "alignment");

// Gate arrays, per token r of a chunk: GA_G the cumulative log2 gate G_r;
// GA_B beta_r; GA_BG beta_r 2^{G_r}; GA_TAIL 2^{G_C - G_r}; GA_OUT
// scale 2^{G_r}; GA_ROW 2^{G_r - G_b}, b the first token of r's 16-token
// block; GA_COL + I - 1 (I = 1, 2, 3): 2^{G_16I - G_r}; GA_END 2^{G_C} (every
// entry).  Off-diagonal 16x16 blocks take 2^{G_i - G_j} as
// GA_ROW[i] * GA_COL[I][j]: both factors lie in [0, 1].
enum { GA_G = 0, GA_B, GA_BG, GA_TAIL, GA_OUT, GA_ROW, GA_COL, GA_END = GA_COL + 3 };
static_assert(GA_END + 1 == NGA, "gate arrays");

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ f32x4 mma32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, a),
                                                     __builtin_bit_cast(bf16x4, b), c, 0, 0, 0);
}
__device__ __forceinline__ u32x2 pk4(f32x4 v) {
    return u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}
__device__ __forceinline__ u32x2 pk4(float4 v) {
    return u32x2{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
}
// two accumulator tiles (rows 4g..4g+3 of each) as one 16x16x32 operand
__device__ __forceinline__ u32x4 pk8(f32x4 lo, f32x4 hi) {
    return u32x4{pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]), pack_bf16x2(hi[0], hi[1]),
                 pack_bf16x2(hi[2], hi[3])};
}
__device__ __forceinline__ u32x4 cat(u32x2 lo, u32x2 hi) { return u32x4{lo[0], lo[1], hi[0], hi[1]}; }
__device__ __forceinline__ f32x4 unpk4(u32x2 w) {
    return f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                 __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u)};
}
// Transposing read of a 16x16 bf16 block: lane j of 16-lane group g passes the
// address of its row 4g + j/4, columns 4(j%4)..+3, and lane 16g+n receives
// X[4g..4g+3][n].
__device__ __forceinline__ u32x2 tr_read(const void* p) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p));
}
__device__ __forceinline__ u32x4 ld16(const char* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x2 ld8(const char* p) { return *reinterpret_cast<const u32x2*>(p); }
__device__ __forceinline__ float4 ldf4(const float* p) { return *reinterpret_cast<const float4*>(p); }

__device__ __forceinline__ int kq_sw(int r) { return K == 128 ? (2 * r) & 14 : r & 6; }
// byte offset of 16-byte group `grp` of row r of a K/Q slot
__device__ __forceinline__ int kq_off(int r, int grp) { return r * 2 * K + ((grp ^ kq_sw(r)) << 4); }

// Inclusive prefix sum over the 64 lanes with DPP row shifts and row
// broadcasts (no LDS traffic).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float add_dpp(float v) {
    return v + __int_as_float(
                   __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}
__device__ __forceinline__ float wave_scan(float x) {
    x = add_dpp<0x111, 0xf>(x);   // row_shr:1
    x = add_dpp<0x112, 0xf>(x);   // row_shr:2
    x = add_dpp<0x114, 0xf>(x);   // row_shr:4
    x = add_dpp<0x118, 0xf>(x);   // row_shr:8
    x = add_dpp<0x142, 0xa>(x);   // row_bcast:15 into rows 1 and 3
    x = add_dpp<0x143, 0xc>(x);   // row_bcast:31 into rows 2 and 3
    return x;
}
__device__ __forceinline__ float lane_of(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Signals between waves: a release store after the data it covers, an
// acquire poll before the data is read.  The poll gives up after a bounded
// number of tries, so a schedule error can never leave a wave that does not
// finish; a poll that gives up sets the caller's status word (`sync_status`,
// never cleared here), so the wrong results it leads to are reported.
typedef __attribute__((address_space(3))) int lds_int;
__device__ __forceinline__ void signal(lds_int* f, int v) {
    __hip_atomic_store(f, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void wait_for(lds_int* f, int v, int* sync_status) {
    for (int it = 0; it < (1 << 16); ++it) {
        if (__hip_atomic_load(f, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= v) return;
        __builtin_amdgcn_s_sleep(1);
    }
    if (sync_status && (threadIdx.x & 63) == 0) atomicOr(sync_status, 1);
}
// Workgroup barrier that waits for this wave's LDS traffic only (loads into
// LDS stay in flight across it; they are covered by signals).
__device__ __forceinline__ void wg_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
}
// buffer loads with the LDS destination: lane l's 16 (or 4) bytes land at
// lds + 16 l (4 l); offsets at or past `bytes` read as zero
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}
__device__ __forceinline__ void to_lds16(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, off, 0, 0, 0);
}
__device__ __forceinline__ void to_lds4(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 4, off, 0, 0, 0);
}
// the same wave reads back what it wrote to LDS
__device__ __forceinline__ void own_lds_sync() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0) only
    __builtin_amdgcn_wave_barrier();
}

struct Ctx {
    char* sm;
    const bf16 *q, *k, *v;
    const float *beta, *g;
    int64_t H, h, t0, len;   // value heads (the state's head), this value head
    int64_t Hq, hq;          // q/k heads, the q/k head this value head reads (GVA)
    int v0, nch, lane, wave;
    float scale;
    Act act;
    float a_log, dt_bias;   // this head's gate-activation parameters
    int* sync_status;       // set when a wait gives up (nullptr: not reported)
    bool loads_first;       // issue each chunk's loads before deriving its gates

    // slot accessors take chunk indices >= 0
    __device__ __forceinline__ char* sK(int c) const { return sm + o_K + SZ_KQ * (c % 3); }
    __device__ __forceinline__ char* sQ(int c) const { return sm + o_Q + SZ_KQ * (c % 3); }
    __device__ __forceinline__ char* sV(int c) const { return sm + o_V + SZ_V * (c % 3); }
    __device__ __forceinline__ char* sRaw(int c) const { return sm + o_RAW + SZ_RAW * (c & 1); }
    __device__ __forceinline__ float* gate(int c, int a) const {
        return reinterpret_cast<float*>(sm + o_G + SZ_G * (c % 3)) + a * C;
    }
    __device__ __forceinline__ char* sAQ(int c) const { return sm + o_AQ + SZ_AQ * (c & 1); }
    __device__ __forceinline__ char* sTT() const { return sm + o_TT; }
    __device__ __forceinline__ char* sA(int c) const { return sm + o_A + SZ_A * (c & 1); }
    __device__ __forceinline__ float* sD(int b) const {
        return reinterpret_cast<float*>(sm + o_D + SZ_DB * b);
    }
    __device__ __forceinline__ char* sDT(int b) const { return sm + o_DT + SZ_DT * b; }
    // squared norms of the current chunk's tokens, per product wave (slot 0:
    // the key wave, 1 + s: query set s)
    __device__ __forceinline__ float* nrm(int slot) const {
        return reinterpret_cast<float*>(sm + o_NRM + SZ_NRM * slot);
    }
    __device__ __forceinline__ lds_int* tflag() const { return (lds_int*)(sm + o_F); }
    __device__ __forceinline__ lds_int* dflag() const { return (lds_int*)(sm + o_F) + 1; }
    __device__ __forceinline__ lds_int* lflag() const { return (lds_int*)(sm + o_F) + 5; }
    // q/k L2 normalisation: the key wave's |k|^2 of the chunk are in nrm(0)
    __device__ __forceinline__ lds_int* nflag() const { return (lds_int*)(sm + o_F) + 6; }

    __device__ __forceinline__ bool valid(int c) const { return c >= 0 && c < nch; }
    __device__ __forceinline__ int rows(int c) const {
        return (int)min((int64_t)C, len - (int64_t)c * C);
    }
    // chunk index clamped into the sequence; an empty sequence (nch = 0)
    // maps to chunk 0, whose row count rows(0) = 0 makes every buffer load
    // of it read zeros without touching memory
    __device__ __forceinline__ int clampc(int c) const { return max(min(c, nch - 1), 0); }
    // byte offset of row r (clamped to the chunk's last row) from the chunk's
    // first row; rows are H*D elements of `eb` bytes apart
    __device__ __forceinline__ uint32_t roff(int c, int r, int D, int eb) const {
        return (uint32_t)min(r, rows(c) - 1) * (uint32_t)(H * D * eb);
    }
    template <typename P>
    __device__ __forceinline__ const char* row0(const P* base, int c, int D) const {
        return reinterpret_cast<const char*>(base + ((t0 + (int64_t)c * C) * H + h) * D);
    }
    // first row of chunk c of q or k (H_q heads)
    __device__ __forceinline__ const char* row0_qk(const bf16* base, int c) const {
        return reinterpret_cast<const char*>(base + ((t0 + (int64_t)c * C) * Hq + hq) * K);
    }
};

// index of the causal 16x16x32 Aqk / T fragment (t, p), p <= t/2
__device__ __forceinline__ constexpr int frag_ix(int t, int p) { return t < 2 ? t : 2 * t - 2 + p; }
// index of the off-diagonal A block (I, J), J < I
__device__ __forceinline__ constexpr int ab_ix(int I, int J) { return I * (I - 1) / 2 + J; }

// q/k L2 normalisation folded into the products (ACT_QK_L2NORM): every
// product is linear in each row, so 1/|x_t| = rsq(x_t.x_t + 1e-6) scales the
// results.  x_t.x_t is the diagonal of a 16x16 Gram tile gt = X_I X_I^T (lane
// 16g+n holds gt[n][4g+e]: row n's diagonal entry sits in lane 16(n/4)+n,
// element n%4), copied to dst[n] by those 16 lanes.
__device__ __forceinline__ void diag_to(float* dst, const f32x4& gt, int lane) {
    const int n = lane & 15, k = n & 3;
    if ((lane >> 4) == (n >> 2)) dst[n] = k == 0 ? gt[0] : k == 1 ? gt[1] : k == 2 ? gt[2] : gt[3];
}
__device__ __forceinline__ float l2_rsq(float xx) { return __builtin_amdgcn_rsqf(xx + L2_EPS); }
__device__ __forceinline__ float4 l2_rsq4(float4 v) {
    return make_float4(l2_rsq(v.x), l2_rsq(v.y), l2_rsq(v.z), l2_rsq(v.w));
}

// ---------------------------------------------------------------- wave 6: loads and gates
__device__ __forceinline__ void role_load(const Ctx& x) {
    const int lane = x.lane;
    const uint32_t skq = (uint32_t)(x.Hq * K * 2), sv = (uint32_t)(x.H * V * 2);
    const uint32_t sg = (uint32_t)(x.H * 4);
    // source offsets inside a chunk: K/Q load s fills rows RPL s .. RPL s +
    // RPL - 1 (lane l: row RPL s + l/GPR, LDS group l%GPR), V load s rows
    // 16s..16s+15 (lane l: row 16s + l/4, LDS group l%4)
    constexpr int RPL = 64 / GPR;
    uint32_t okq[GPR], ov[4];
#pragma unroll
    for (int s = 0; s < GPR; ++s) {
        const int r = RPL * s + lane / GPR;
        okq[s] = (uint32_t)r * skq + 16u * (uint32_t)((lane % GPR) ^ kq_sw(r));
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int r = 16 * s + (lane >> 2);
        ov[s] = (uint32_t)r * sv + (uint32_t)x.v0 * 2 + 16u * (uint32_t)((lane & 3) ^ (2 * ((r >> 2) & 1)));
    }
    const uint32_t lg = (uint32_t)lane * sg;
    // g and beta of chunk c into raw slot c (rows past a ragged end read as 0)
    auto load_raw = [&](int c) __attribute__((always_inline)) {
        const int cc = x.clampc(c);
        const uint32_t nb = (uint32_t)x.rows(cc) * sg;
        to_lds4(rsrc(x.row0(x.g, cc, 1), nb), x.sRaw(c), lg);
        to_lds4(rsrc(x.row0(x.beta, cc, 1), nb), x.sRaw(c) + C * 4, lg);
    };
    load_raw(0);
    for (int j = -2; j < x.nch; ++j) {
        // everything started an iteration ago has landed: K, Q, V of chunk j+1
        // (signalled to the product waves) and g, beta of chunk j+2
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
        signal(x.lflag(), j + 2);
        const int c2 = j + 2;
        // gate arrays of chunk j+2, read from the next iteration on
        auto gates = [&]() __attribute__((always_inline)) {
            if (x.valid(c2)) {
                const float* raw = reinterpret_cast<const float*>(x.sRaw(c2));
                float gl = raw[lane], bt = raw[C + lane];
                if (x.act.flags) {
                    // raw logits: rows past a ragged end must stay g = 0, beta = 0
                    const bool in = lane < x.rows(c2);
                    if (x.act.flags & ACT_GATE) gl = in ? act_log_gate(gl, x.a_log, x.dt_bias) : 0.f;
                    if (x.act.flags & ACT_BETA_SIGMOID)
                        bt = in ? act_beta(bt, x.act.flags & ACT_BETA_NEG_EIG) : 0.f;
                }
                const float G = wave_scan(gl * LOG2E);
                const float Gc = lane_of(G, C - 1);
                const float gam = exp2_hw(G);
                x.gate(c2, GA_G)[lane] = G;
                x.gate(c2, GA_B)[lane] = bt;
                x.gate(c2, GA_BG)[lane] = bt * gam;
                x.gate(c2, GA_TAIL)[lane] = exp2_hw(fminf(Gc - G, 0.f));
                x.gate(c2, GA_OUT)[lane] = x.scale * gam;
                float Gs[4];
#pragma unroll
                for (int I = 0; I < 4; ++I) Gs[I] = lane_of(G, 16 * I);
                const int bl = lane >> 4;
                const float Gb = bl == 0 ? Gs[0] : bl == 1 ? Gs[1] : bl == 2 ? Gs[2] : Gs[3];
                x.gate(c2, GA_ROW)[lane] = exp2_hw(fminf(G - Gb, 0.f));
#pragma unroll
                for (int I = 1; I < 4; ++I)
                    x.gate(c2, GA_COL + I - 1)[lane] = exp2_hw(fminf(Gs[I] - G, 0.f));
                x.gate(c2, GA_END)[lane] = exp2_hw(Gc);
            }
        };
        auto issue = [&]() __attribute__((always_inline)) {
            // start the loads of K, Q, V of chunk j+2 and g, beta of chunk j+3 (a
            // clamped duplicate past the end: its slot is free either way)
            const int ck = x.clampc(c2);
            const uint32_t nr = (uint32_t)x.rows(ck);
            const __amdgpu_buffer_rsrc_t rk = rsrc(x.row0_qk(x.k, ck), nr * skq);
            const __amdgpu_buffer_rsrc_t rq = rsrc(x.row0_qk(x.q, ck), nr * skq);
            const __amdgpu_buffer_rsrc_t rv = rsrc(x.row0(x.v, ck, V), nr * sv);
#pragma unroll
            for (int s = 0; s < GPR; ++s) {
                to_lds16(rk, x.sK(c2) + 1024 * s, okq[s]);
                to_lds16(rq, x.sQ(c2) + 1024 * s, okq[s]);
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) to_lds16(rv, x.sV(c2) + 1024 * s, ov[s]);
            load_raw(j + 3);
        };
        // Inputs larger than the Infinity Cache come from HBM: their loads
        // are issued first, which gives them the whole step to land.  Cache
        // hits land early enough either way, and issued after the gate arrays
        // their LDS writes meet less of the state waves' first reads.
        if (x.loads_first) {
            issue();
            gates();
        } else {
            gates();
            issue();
        }
        wg_barrier();
    }
    // no load may land in LDS after the workgroup has ended
    __builtin_amdgcn_s_waitcnt(0x0F70);
}

// ---------------------------------------------------------------- waves 3,4,5,7: masked products
// Blocks (I, J) of chunk c: lane 16g+n of each result holds S[16I+n][16J+4g+e]
// (row 16I+n, key column 16J+4g+e), with A = K_J rows and B = K_I or Q_I rows.

// wave 3: A = beta_i 2^{G_i - G_j} k_i.k_j, the four diagonal blocks first
// (signalled to the inverse), then the six below them
template <bool L2>
__device__ __forceinline__ void role_keys(const Ctx& x) {
    const int lane = x.lane, m = lane & 15, g = lane >> 4;
    for (int j = -2; j < x.nch; ++j) {
        const int c = j + 1;
        if (x.valid(c)) {
            wait_for(x.lflag(), c + 1, x.sync_status);   // K, Q of chunk c have landed
            const char* kb = x.sK(c);
            u32x4 kf[4][NKK];
#pragma unroll
            for (int I = 0; I < 4; ++I)
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) kf[I][kk] = ld16(kb + kq_off(16 * I + m, 4 * kk + g));
            float Gi[4], bi[4];
            float4 Gj[4];
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                Gi[I] = x.gate(c, GA_G)[16 * I + m];
                bi[I] = x.gate(c, GA_B)[16 * I + m];
                Gj[I] = ldf4(x.gate(c, GA_G) + 16 * I + 4 * g);
            }
            __builtin_amdgcn_sched_barrier(0);
            f32x4 sd[4];
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                sd[I] = zero4();
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) sd[I] = mma32(kf[I][kk], kf[I][kk], sd[I]);
            }
            // q/k L2 normalisation: 1/|k| of the rows (16I+m) and columns
            // (16I+4g+e) of the diagonal blocks, from their own diagonals
            constexpr bool l2 = L2;
            float rkr[4] = {1.f, 1.f, 1.f, 1.f};
            float4 rkc[4];
#pragma unroll
            for (int I = 0; I < 4; ++I) rkc[I] = make_float4(1.f, 1.f, 1.f, 1.f);
            float* nk = x.nrm(0);
            if constexpr (l2) {
#pragma unroll
                for (int I = 0; I < 4; ++I) diag_to(nk + 16 * I, sd[I], lane);
                own_lds_sync();
                signal(x.nflag(), c + 1);   // the query waves read them too
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    rkr[I] = l2_rsq(nk[16 * I + m]);
                    rkc[I] = l2_rsq4(ldf4(nk + 16 * I + 4 * g));
                }
#pragma unroll
                for (int I = 0; I < 4; ++I)
#pragma unroll
                    for (int e = 0; e < 4; ++e) sd[I][e] *= rkr[I] * (&rkc[I].x)[e];
            }
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                float4 ad;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    (&ad.x)[e] = 4 * g + e < m ? bi[I] * exp2_hw(fminf(Gi[I] - (&Gj[I].x)[e], 0.f)) * sd[I][e]
                                               : 0.f;
                *reinterpret_cast<float4*>(x.sD(I) + m * LDD + 4 * g) = ad;
            }
            signal(x.dflag(), c + 1);
            // off-diagonal blocks: decay ROW[i] COL_I[j]
#pragma unroll
            for (int I = 1; I < 4; ++I) {
                const float bri = bi[I] * x.gate(c, GA_ROW)[16 * I + m];
                const float* colI = x.gate(c, GA_COL + I - 1);
#pragma unroll
                for (int J = 0; J < I; ++J) {
                    f32x4 s = zero4();
#pragma unroll
                    for (int kk = 0; kk < NKK; ++kk) s = mma32(kf[J][kk], kf[I][kk], s);
                    const float4 cj = ldf4(colI + 16 * J + 4 * g);
                    f32x4 av;
                    if constexpr (l2) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) s[e] *= rkr[I] * (&rkc[J].x)[e];
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) av[e] = bri * (&cj.x)[e] * s[e];
                    *reinterpret_cast<u32x2*>(x.sA(c) + ab_ix(I, J) * SZ_AB + m * (LDAB * 2) + 8 * g) =
                        pk4(av);
                }
            }
            if constexpr (l2) {   // the state pass's K h and K^T V_new rows: 1/|k| into beta gamma and the tail
                const float rk = l2_rsq(nk[lane]);
                x.gate(c, GA_BG)[lane] *= rk;
                x.gate(c, GA_TAIL)[lane] *= rk;
            }
        }
        wg_barrier();
    }
}

// waves 7, 4, 5: Aqk = scale 2^{G_i - G_j} q_i.k_j (j <= i), as the state
// pass's 16x16x32 operand fragments.  Set 0 takes the diagonal blocks and
// (1,0), set 1 (2,0) and (2,1), set 2 (3,0), (3,1) and (3,2).  With q/k L2
// normalisation each set also forms the Q Q^T diagonal blocks of its block
// rows, so the sets split by block row instead (set 0 rows 0-1, set 1 row 2,
// set 2 row 3) and each folds 1/|q| of its own rows into the output's scale.
template <int SET, bool L2>
__device__ __forceinline__ void role_queries(const Ctx& x) {
    constexpr int NB = L2 ? (SET == 2 ? 4 : 3) : SET == 0 ? 5 : SET == 1 ? 2 : 3;
    constexpr int BI[3][5] = {{0, 1, L2 ? 1 : 2, 3, 1}, {2, 2, 2, 0, 0}, {3, 3, 3, 3, 0}};
    constexpr int BJ[3][5] = {{0, 1, L2 ? 0 : 2, 3, 0}, {0, 1, 2, 0, 0}, {0, 1, 2, 3, 0}};
    const int lane = x.lane, m = lane & 15, g = lane >> 4;
    for (int j = -2; j < x.nch; ++j) {
        const int c = j + 1;
        if (x.valid(c)) {
            wait_for(x.lflag(), c + 1, x.sync_status);   // K, Q of chunk c have landed
            const char* kb = x.sK(c);
            const char* qb = x.sQ(c);
            u32x4 kf[4][NKK], qf[4][NKK];
            bool needk[4] = {false, false, false, false}, needq[4] = {false, false, false, false};
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                needk[BJ[SET][b]] = true;
                needq[BI[SET][b]] = true;
            }
#pragma unroll
            for (int J = 0; J < 4; ++J)
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) {
                    if (needk[J]) kf[J][kk] = ld16(kb + kq_off(16 * J + m, 4 * kk + g));
                    if (needq[J]) qf[J][kk] = ld16(qb + kq_off(16 * J + m, 4 * kk + g));
                }
            __builtin_amdgcn_sched_barrier(0);
            // q/k L2 normalisation: 1/|q| of the rows of the blocks' I from
            // the diagonals of their Q Q^T blocks, 1/|k| of the columns of
            // their J from the key wave's K K^T diagonals
            constexpr bool l2 = L2;
            float rqr[4] = {1.f, 1.f, 1.f, 1.f};
            float4 rkc[4];
#pragma unroll
            for (int J = 0; J < 4; ++J) rkc[J] = make_float4(1.f, 1.f, 1.f, 1.f);
            if constexpr (l2) {
                float* nq = x.nrm(1 + SET);   // [64, 128): |q|^2
#pragma unroll
                for (int J = 0; J < 4; ++J) {
                    if (needq[J]) {
                        f32x4 gq = zero4();
#pragma unroll
                        for (int kk = 0; kk < NKK; ++kk) gq = mma32(qf[J][kk], qf[J][kk], gq);
                        diag_to(nq + 64 + 16 * J, gq, lane);
                    }
                }
                own_lds_sync();
                wait_for(x.nflag(), c + 1, x.sync_status);
                const float* nk = x.nrm(0);
#pragma unroll
                for (int J = 0; J < 4; ++J) {
                    if (needk[J]) rkc[J] = l2_rsq4(ldf4(nk + 16 * J + 4 * g));
                    if (needq[J]) rqr[J] = l2_rsq(nq[64 + 16 * J + m]);
                }
                // 1/|q| of this set's rows into the output's scale gamma
                if (needq[lane >> 4]) x.gate(c, GA_OUT)[lane] *= l2_rsq(nq[64 + lane]);
            }
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int I = BI[SET][b], J = BJ[SET][b];
                f32x4 s = zero4();
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) s = mma32(kf[J][kk], qf[I][kk], s);
                if constexpr (l2) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) s[e] *= rqr[I] * (&rkc[J].x)[e];
                }
                f32x4 q;
                if (J == I) {
                    const float Gi = x.gate(c, GA_G)[16 * I + m];
                    const float4 Gj = ldf4(x.gate(c, GA_G) + 16 * I + 4 * g);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        q[e] = 4 * g + e <= m ? x.scale * exp2_hw(fminf(Gi - (&Gj.x)[e], 0.f)) * s[e] : 0.f;
                } else {
                    const float sri = x.scale * x.gate(c, GA_ROW)[16 * I + m];
                    const float4 cj = ldf4(x.gate(c, GA_COL + I - 1) + 16 * J + 4 * g);
#pragma unroll
                    for (int e = 0; e < 4; ++e) q[e] = sri * (&cj.x)[e] * s[e];
                }
                *reinterpret_cast<u32x2*>(x.sAQ(c) + frag_ix(I, J >> 1) * 1024 + lane * 16 +
                                          8 * (J & 1)) = pk4(q);
            }
        }
        wg_barrier();
    }
}

// ---------------------------------------------------------------- wave 2: the inverse
// T^T in LDS: row c holds column c of T (bf16, LDTT per row).
// TT block (I, J) of T, from an accumulator tile holding T_IJ[4g+e][n]:
__device__ __forceinline__ void put_tt(char* tt, int I, int J, int lane, f32x4 v) {
    *reinterpret_cast<u32x2*>(tt + ((16 * J + (lane & 15)) * LDTT + 16 * I + 4 * (lane >> 4)) * 2) =
        pk4(v);
}
// 16x16x16 A operand of T_bb (lane 16g+m: T_bb[m][4g..4g+3])
__device__ __forceinline__ u32x2 tt_a(const char* tt, int b, int lane) {
    const int g = lane >> 4, jl = lane & 15;
    return tr_read(tt + ((16 * b + 4 * g + (jl >> 2)) * LDTT + 16 * b + 4 * (jl & 3)) * 2);
}
// 16x16x16 A operand of the off-diagonal A block (I, J)
__device__ __forceinline__ u32x2 ab_a(const char* a, int I, int J, int lane) {
    return ld8(a + ab_ix(I, J) * SZ_AB + (lane & 15) * (LDAB * 2) + 8 * (lane >> 4));
}
__device__ __forceinline__ u32x2 neg4(f32x4 v) { return pk4(-v); }

// T_j from the diagonal-block inverses tbb (accumulator tiles) and the
// off-diagonal A blocks
__device__ __forceinline__ void compose(const Ctx& x, int j, const f32x4 (&tbb)[4]) {
    const int lane = x.lane;
    char* tt = x.sTT();
#pragma unroll
    for (int b = 0; b < 4; ++b) put_tt(tt, b, b, lane, tbb[b]);
    const char* a = x.sA(j);
    const u32x2 a10 = ab_a(a, 1, 0, lane), a20 = ab_a(a, 2, 0, lane), a21 = ab_a(a, 2, 1, lane);
    const u32x2 a30 = ab_a(a, 3, 0, lane), a31 = ab_a(a, 3, 1, lane), a32 = ab_a(a, 3, 2, lane);
    const u32x2 t00 = pk4(tbb[0]), t11 = pk4(tbb[1]), t22 = pk4(tbb[2]);
    // products that need only the diagonal inverses
    const f32x4 y1 = mma16(a10, t00, zero4());     // A10 T00
    const f32x4 x32 = mma16(a32, t22, zero4());    // A32 T22
    const f32x4 y01 = mma16(a21, t11, zero4());    // A21 T11
    const f32x4 y11 = mma16(a31, t11, zero4());    // A31 T11
    f32x4 y00 = mma16(a20, t00, zero4());          // A20 T00 + ...
    f32x4 y10 = mma16(a30, t00, zero4());          // A30 T00 + ...
    own_lds_sync();                                // the diagonal blocks of T^T are in LDS
    const u32x2 t11a = tt_a(tt, 1, lane), t22a = tt_a(tt, 2, lane), t33a = tt_a(tt, 3, lane);
    const f32x4 t10 = mma16(t11a, neg4(y1), zero4());    // T10 = -T11 A10 T00
    const f32x4 t32 = mma16(t33a, neg4(x32), zero4());   // T32 = -T33 A32 T22
    const f32x4 t21 = mma16(t22a, neg4(y01), zero4());   // T21 = -T22 A21 T11
    const u32x2 t10b = pk4(t10);
    y00 = mma16(a21, t10b, y00);                         // A20 T00 + A21 T10
    y10 = mma16(a31, t10b, y10);                         // A30 T00 + A31 T10
    const f32x4 w11 = mma16(a32, pk4(t21), y11);         // A31 T11 + A32 T21
    const f32x4 t20 = mma16(t22a, neg4(y00), zero4());   // T20 = -T22 (A20 T00 + A21 T10)
    const f32x4 t31 = mma16(t33a, neg4(w11), zero4());   // T31 = -T33 (A31 T11 + A32 T21)
    const f32x4 w10 = mma16(a32, pk4(t20), y10);         // A30 T00 + A31 T10 + A32 T20
    const f32x4 t30 = mma16(t33a, neg4(w10), zero4());   // T30
    put_tt(tt, 1, 0, lane, t10);
    put_tt(tt, 3, 2, lane, t32);
    put_tt(tt, 2, 1, lane, t21);
    put_tt(tt, 2, 0, lane, t20);
    put_tt(tt, 3, 1, lane, t31);
    put_tt(tt, 3, 0, lane, t30);
    signal(x.tflag(), j + 1);
}

// Inverses of the four 16x16 diagonal blocks of I + A of chunk c, as
// accumulator tiles (lane 16g+n: T_bb[4g+e][n]).
__device__ __forceinline__ void diag_inverse(const Ctx& x, f32x4 (&tbb)[4]) {
    const int lane = x.lane;
    // forward substitution of the 8x8 block s of 16x16 block b, column c
    {
        const int b = lane >> 4, s = (lane >> 3) & 1, col = lane & 7;
        const float* d = x.sD(b) + 8 * s * LDD + 8 * s;
        float4 rw[8][2];
#pragma unroll
        for (int i = 1; i < 8; ++i) {
            rw[i][0] = ldf4(d + i * LDD);
            rw[i][1] = ldf4(d + i * LDD + 4);
        }
        float xv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float acc = i == col ? 1.f : 0.f;
#pragma unroll
            for (int mm = 0; mm < i; ++mm)
                acc -= (mm < 4 ? (&rw[i][0].x)[mm] : (&rw[i][1].x)[mm - 4]) * xv[mm];
            xv[i] = acc;
        }
        // row (8s + col) of D_b^T: column 8s+col of D_b, zero outside block s
        const u32x2 w0{pack_bf16x2(xv[0], xv[1]), pack_bf16x2(xv[2], xv[3])};
        const u32x2 w1{pack_bf16x2(xv[4], xv[5]), pack_bf16x2(xv[6], xv[7])};
        const u32x2 z{0u, 0u};
        char* dt = x.sDT(b) + (8 * s + col) * (LDDT * 2);
        *reinterpret_cast<u32x2*>(dt) = s ? z : w0;
        *reinterpret_cast<u32x2*>(dt + 8) = s ? z : w1;
        *reinterpret_cast<u32x2*>(dt + 16) = s ? w0 : z;
        *reinterpret_cast<u32x2*>(dt + 24) = s ? w1 : z;
    }
    own_lds_sync();
    // T_bb = D - D (X D), X = the lower-left 8x8 block of A_bb.  The reads of
    // all four blocks are issued first (every lane's addresses lie inside
    // the blocks; lanes outside X only zero their value), so the four
    // blocks cost one LDS latency, not three each.
    const int g = lane >> 4, mrow = lane & 15;
    const bool live = mrow >= 8 && g < 2;
    float4 xr[4];
    u32x2 db[4], da[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        xr[b] = ldf4(x.sD(b) + mrow * LDD + 4 * g);
        db[b] = ld8(x.sDT(b) + mrow * (LDDT * 2) + 8 * g);   // D[4g+e][n], n = lane & 15
        da[b] = tr_read(x.sDT(b) + (4 * g + (mrow >> 2)) * (LDDT * 2) + 8 * (mrow & 3));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const u32x2 xa = live ? pk4(xr[b]) : u32x2{0u, 0u};
        const f32x4 y = mma16(xa, db[b], zero4());
        tbb[b] = mma16(da[b], neg4(y), unpk4(db[b]));
    }
}

__device__ __forceinline__ void role_inverse(const Ctx& x) {
    f32x4 tbb[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) tbb[b] = zero4();
    for (int j = -2; j < x.nch; ++j) {
        if (x.valid(j)) compose(x, j, tbb);
        const int c = j + 1;
        if (x.valid(c)) {
            wait_for(x.dflag(), c + 1, x.sync_status);   // the diagonal blocks of A
            diag_inverse(x, tbb);
        }
        wg_barrier();
    }
}

// ---------------------------------------------------------------- waves 0,1: the state pass
__device__ __forceinline__ void role_state(const Ctx& x, const FusedLaunch& a, int64_t n) {
    __builtin_amdgcn_s_setprio(2);
    const int lane = x.lane, m = lane & 15, g = lane >> 4;
    const int n0 = 16 * x.wave;
    const int64_t hbase = (n * a.H + x.h) * (int64_t)(K * V) + x.v0 + n0 + m;
    // row 4g+e of state tile r is key channel 32(r/2) + 8g + 4(r%2) + e
    auto chan = [&](int r, int e) { return 32 * (r >> 1) + 8 * g + 4 * (r & 1) + e; };
    f32x4 hacc[NST];
#pragma unroll
    for (int r = 0; r < NST; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            hacc[r][e] = a.h0 ? a.h0[hbase + (int64_t)chan(r, e) * V] : 0.f;
    bf16* o = static_cast<bf16*>(a.o);

    for (int j = -2; j < x.nch; ++j) {
        if (x.valid(j)) {
            const char* kb = x.sK(j);
            const char* qb = x.sQ(j);
            // h as 16x16x32 operands: key channels 32kk+8g..+7 of column m
            u32x4 hb[NKK];
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) hb[kk] = pk8(hacc[2 * kk], hacc[2 * kk + 1]);
            // The reads of each step are issued in batches ahead of the
            // products that use them (scheduling barriers keep the compiler
            // from sinking them next to their uses, which would expose one LDS
            // latency per product).
            // ---- X = K h (token rows 16t+4g+e, column m) and (Q h)^T (column
            // 4g+e, token 16t+m)
            u32x4 kf[NKK][4], qf[NKK][4];
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    kf[kk][t] = ld16(kb + kq_off(16 * t + m, 4 * kk + g));
                    qf[kk][t] = ld16(qb + kq_off(16 * t + m, 4 * kk + g));
                }
                if (kk == NKK / 2 - 1) __builtin_amdgcn_sched_barrier(0);
            }
            f32x4 xa[4], oa[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) xa[t] = oa[t] = zero4();
#pragma unroll
            for (int kk = 0; kk < NKK / 2; ++kk)
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    xa[t] = mma32(kf[kk][t], hb[kk], xa[t]);
                    oa[t] = mma32(hb[kk], qf[kk][t], oa[t]);
                }
            __builtin_amdgcn_sched_barrier(0);
            // V rows 16t+4g+e, column n0+m (the accumulator's layout), and the
            // gates of R
            const float* gb = x.gate(j, GA_B);
            const float* gbg = x.gate(j, GA_BG);
            u32x2 vr[4];
            float4 b4[4], bg4[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int r = 16 * t + 4 * g + (m >> 2);
                const int q = (2 * x.wave + ((m & 3) >> 1)) ^ (2 * ((r >> 2) & 1));
                vr[t] = tr_read(x.sV(j) + r * (VT * 2) + 16 * q + 8 * (m & 1));
                b4[t] = ldf4(gb + 16 * t + 4 * g);
                bg4[t] = ldf4(gbg + 16 * t + 4 * g);
            }
#pragma unroll
            for (int kk = NKK / 2; kk < NKK; ++kk)
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    xa[t] = mma32(kf[kk][t], hb[kk], xa[t]);
                    oa[t] = mma32(hb[kk], qf[kk][t], oa[t]);
                }
            __builtin_amdgcn_sched_barrier(0);
            // ---- R = beta V - beta gamma X
            u32x4 rb[2];
            f32x4 rt[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const f32x4 vv = unpk4(vr[t]);
#pragma unroll
                for (int e = 0; e < 4; ++e) rt[t][e] = (&b4[t].x)[e] * vv[e] - (&bg4[t].x)[e] * xa[t][e];
            }
#pragma unroll
            for (int p = 0; p < 2; ++p) rb[p] = pk8(rt[2 * p], rt[2 * p + 1]);
            // ---- V_new = T R; the later steps' operands are read meanwhile
            wait_for(x.tflag(), j + 1, x.sync_status);
            const char* tt = x.sTT();
            u32x4 tf[4][2];
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    if (2 * p > t) continue;
                    const char* base = tt + ((32 * p + 4 * g + (m >> 2)) * LDTT + 16 * t + 4 * (m & 3)) * 2;
                    tf[t][p] = cat(tr_read(base), tr_read(base + 16 * LDTT * 2));
                }
            const float* gtl = x.gate(j, GA_TAIL);
            const float* gout = x.gate(j, GA_OUT);
            const char* aq = x.sAQ(j);
            float4 tl[4];
            float so[4];
            u32x4 af[4][2];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                tl[t] = ldf4(gtl + 16 * t + 4 * g);
                so[t] = gout[16 * t + m];
#pragma unroll
                for (int p = 0; p < 2; ++p)
                    if (2 * p <= t) af[t][p] = ld16(aq + frag_ix(t, p) * 1024 + lane * 16);
            }
            const float gC = x.gate(j, GA_END)[0];
            __builtin_amdgcn_sched_barrier(0);
            f32x4 va[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                va[t] = zero4();
#pragma unroll
                for (int p = 0; p < 2; ++p)
                    if (2 * p <= t) va[t] = mma32(tf[t][p], rb[p], va[t]);
            }
            // decayed V_new for the state, V_new for the output
            u32x4 vsb[2], vnb[2];
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                f32x4 s0, s1;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    s0[e] = (&tl[2 * p].x)[e] * va[2 * p][e];
                    s1[e] = (&tl[2 * p + 1].x)[e] * va[2 * p + 1][e];
                }
                vsb[p] = pk8(s0, s1);
                vnb[p] = pk8(va[2 * p], va[2 * p + 1]);
            }
            // ---- h <- gamma_C h + K^T (decayed V_new): K^T operand by
            // transposing reads of token rows {32p+4g.., 32p+16+4g..}; lane j of
            // a 16-lane group addresses channels 32(r/2) + 8(j%4) + 4(r%2)..+3,
            // i.e. the channels of state tile r's rows 4(j%4)..+3
            u32x4 kt[NST][2];
#pragma unroll
            for (int r = 0; r < NST; ++r) {
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    const int r0 = 32 * p + 4 * g + (m >> 2), r1 = r0 + 16;
                    const int grp = 4 * (r >> 1) + (m & 3), hf = 8 * (r & 1);
                    kt[r][p] = cat(tr_read(kb + kq_off(r0, grp) + hf), tr_read(kb + kq_off(r1, grp) + hf));
                }
                if (r == NST / 2 - 1) __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int r = 0; r < NST; ++r) {
                hacc[r] *= gC;
#pragma unroll
                for (int p = 0; p < 2; ++p) hacc[r] = mma32(kt[r][p], vsb[p], hacc[r]);
                if (r == NST / 2 - 1) __builtin_amdgcn_sched_barrier(0);
            }
            // ---- O^T = diag(scale gamma) (Q h)^T + V_new^T Aqk^T, stored from registers
            const int ntok = x.rows(j);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                oa[t] *= so[t];
#pragma unroll
                for (int p = 0; p < 2; ++p)
                    if (2 * p <= t) oa[t] = mma32(vnb[p], af[t][p], oa[t]);
                const int tok = 16 * t + m;
                if (tok < ntok)
                    // non-temporal: o is not read again here
                    __builtin_nontemporal_store(
                        pk4(oa[t]), reinterpret_cast<u32x2*>(o + ((x.t0 + (int64_t)j * C + tok) * x.H +
                                                                  x.h) * V + x.v0 + n0 + 4 * g));
            }
        }
        wg_barrier();
    }
    if (a.ht)
#pragma unroll
        for (int r = 0; r < NST; ++r)
#pragma unroll
            for (int e = 0; e < 4; ++e) a.ht[hbase + (int64_t)chan(r, e) * V] = hacc[r][e];
}

// ---------------------------------------------------------------- the kernel
template <bool L2>
__global__ __launch_bounds__(NT) void fused_kernel(FusedLaunch a) {
    __shared__ __attribute__((aligned(16))) char smem[L2 ? BYTES_L2 : BYTES];
    const int64_t bid = blockIdx.x;
    // the four value slices of a (sequence, head) run on one XCD (workgroups
    // are dealt to the eight XCDs round-robin), where they share K, Q in L2
    const int vt = (int)((bid >> 3) % NVT);
    const int64_t chain = (bid & 7) + 8 * ((bid >> 3) / NVT);
    if (chain >= a.N * a.H) return;

    Ctx x;
    x.sm = smem;
    x.q = static_cast<const bf16*>(a.q);
    x.k = static_cast<const bf16*>(a.k);
    x.v = static_cast<const bf16*>(a.v);
    x.beta = a.beta;
    x.g = a.g;
    x.H = a.H;
    // packed input: chains longest sequence first (rank order from the table)
    const int64_t r = chain / a.H;
    const int64_t n = a.seqs ? (int64_t)a.seqs[r].w : r;
    x.h = chain - r * a.H;
    x.Hq = a.Hq > 0 ? a.Hq : a.H;
    x.hq = x.h / (a.H / x.Hq);
    x.v0 = vt * VT;
    x.lane = threadIdx.x & 63;
    x.wave = wave_id();
    x.scale = a.scale;
    x.act = a.act;
    x.sync_status = a.sync_status;
    x.loads_first = a.loads_first;
    x.a_log = (a.act.flags & ACT_GATE) ? a.act.A_log[x.h] : 0.f;
    x.dt_bias = (a.act.flags & ACT_GATE) ? a.act.dt_bias[x.h] : 0.f;
    if (a.seqs) {
        const int4 s = a.seqs[n];
        x.t0 = s.x;
        x.len = s.y;
    } else {
        x.t0 = n * a.T;
        x.len = a.T;
    }
    x.nch = (int)((x.len + C - 1) / C);

    // Aqk fragments and T^T start zero: their blocks above the diagonal are
    // read as zeros and never written
    for (int i = threadIdx.x; i < (2 * SZ_AQ + SZ_TT) / 16; i += NT)
        reinterpret_cast<u32x4*>(smem + o_AQ)[i] = u32x4{0u, 0u, 0u, 0u};
    if (threadIdx.x < 16) reinterpret_cast<int*>(smem + o_F)[threadIdx.x] = 0;
    __syncthreads();

    // waves w and w+4 share a SIMD: the two state waves (60 MFMAs per chunk
    // each) pair with the lightest product waves (8 and 12 MFMAs), the
    // inverse (latency-bound) with the loads, the two heaviest product waves
    // (40 and 20) with each other
    switch (x.wave) {
        case 0:
        case 1: role_state(x, a, n); break;
        case 2: role_inverse(x); break;
        case 6: role_load(x); break;
        case 3: role_keys<L2>(x); break;
        case 7: role_queries<0, L2>(x); break;
        case 4: role_queries<1, L2>(x); break;
        default: role_queries<2, L2>(x); break;
    }
}
