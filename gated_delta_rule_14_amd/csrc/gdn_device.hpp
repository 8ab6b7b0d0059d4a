// Device-side helpers shared by the gfx950 kernels: element types, bf16
// conversion, the 16x16 MFMA fragments and small wave utilities.
//
// MFMA fragment layouts used throughout (wave64, 16x16 output tile):
//   bf16 v_mfma_f32_16x16x32_bf16: lane l holds A[l%16][8*(l/16) + 0..7] and
//       B[8*(l/16) + 0..7][l%16]; the f32x4 result holds C[4*(l/16) + 0..3][l%16].
//   f32  v_mfma_f32_16x16x4_f32:   lane l holds A[l%16][l/16] and
//       B[l/16][l%16]; the result layout is the same as above.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

struct bf16 {  // storage-only 16-bit brain float
    uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// Two floats to packed bf16 (lo in bits 0-15), round-to-nearest-even, one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2v v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return (uint16_t)(pack_bf16x2(f, 0.f) & 0xffffu);
}

// element traits: loads/stores of the q/k/v/o element type through float
template <typename T> struct Elem;
// Raw / load_raw / from_raw split a load from its conversion, so that a value
// loaded well ahead of its use is not waited for at the load.
template <> struct Elem<float> {
    static constexpr int BYTES = 4;
    typedef float Raw;
    __device__ __forceinline__ static float load(const float* p) { return *p; }
    __device__ __forceinline__ static Raw load_raw(const float* p) { return *p; }
    __device__ __forceinline__ static float from_raw(Raw r) { return r; }
    __device__ __forceinline__ static void store(float* p, float x) { *p = x; }
};
template <> struct Elem<bf16> {
    static constexpr int BYTES = 2;
    typedef uint32_t Raw;   // the 16 payload bits, zero-extended
    __device__ __forceinline__ static float load(const bf16* p) { return bf16_to_f32(p->bits); }
    __device__ __forceinline__ static Raw load_raw(const bf16* p) { return p->bits; }
    __device__ __forceinline__ static float from_raw(Raw r) { return __uint_as_float(r << 16); }
    __device__ __forceinline__ static void store(bf16* p, float x) { p->bits = f32_to_bf16(x); }
};

// A 16-byte vector of T held in a uint4: element access and packing.
template <typename T> struct Vec16;
template <> struct Vec16<bf16> {
    static constexpr int N = 8;
    __device__ __forceinline__ static float get(const uint4& v, int e) {
        const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
        return bf16_to_f32((uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu)));
    }
    __device__ __forceinline__ static uint4 pack(const float* f) {
        return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                          pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
    }
};
template <> struct Vec16<float> {
    static constexpr int N = 4;
    __device__ __forceinline__ static float get(const uint4& v, int e) {
        return __uint_as_float(e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w);
    }
    __device__ __forceinline__ static uint4 pack(const float* f) {
        return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                          __float_as_uint(f[3]));
    }
};

// 2^x with the hardware exponential (one instruction, about 1 ulp).  Every
// argument here is a log2 decay <= 0, so the result lies in [0, 1]; results
// below the smallest normal float may flush to zero.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Index of the calling wave in its workgroup, in a scalar register: branches
// on it are then taken per wave instead of being masked lane by lane.
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// MFMA fragments.  `row` points at element (row l%16, k0) of a row-major A
// tile, or at (col l%16, k0) of a B^T tile (B stored n-major, k contiguous);
// load() picks this lane's k-slice.  bf16 slices are 16 bytes and must be
// 16-byte aligned.
template <typename T> struct Mma;

template <> struct Mma<bf16> {
    typedef bf16x8 frag;
    static constexpr int KSTEP = 32;  // k covered by one instruction
    __device__ __forceinline__ static frag load(const bf16* row, int lane) {
        return *reinterpret_cast<const bf16x8*>(row + 8 * (lane >> 4));
    }
    // Fragment of a k-major tile X[k][m] (m contiguous, pitch ld elements,
    // `x` at element (k0, m0)): lane 16g+i receives X[k0+8g .. +7][m0+i].
    // Two ds_read_b64_tr_b16: inside each 16-lane group, lane i's element e
    // comes from the 4-element chunk addressed by lane 4e + i/4, position
    // i%4, so lane j addresses row k0+8g+(j>>2) (+4), columns 4(j&3)..+3.
    __device__ __forceinline__ static frag load_t(const bf16* x, int ld, int lane) {
        const int g = lane >> 4, j = lane & 15;
        const bf16* p = x + (8 * g + (j >> 2)) * ld + 4 * (j & 3);
        typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * ld));
        typedef short i16x8 __attribute__((ext_vector_type(8)));
        const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_bit_cast(bf16x8, v);
    }
    __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

template <> struct Mma<float> {
    typedef float frag;
    static constexpr int KSTEP = 4;
    __device__ __forceinline__ static frag load(const float* row, int lane) {
        return row[lane >> 4];
    }
    // k-major tile X[k][m]: lane l receives X[k0 + l/16][m0 + l%16]
    __device__ __forceinline__ static frag load_t(const float* x, int ld, int lane) {
        return x[(lane >> 4) * ld + (lane & 15)];
    }
    __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// Four consecutive elements of T: their raw 8 (bf16) or 16 (fp32) bytes, one
// load, and the floats they hold.
template <typename T> struct Quad;
template <> struct Quad<bf16> {
    typedef u32x2 raw;
    __device__ __forceinline__ static raw load(const bf16* p) {
        return *reinterpret_cast<const u32x2*>(p);
    }
    __device__ __forceinline__ static f32x4 get(raw r) {
        return f32x4{__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                     __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u)};
    }
};
template <> struct Quad<float> {
    typedef u32x4 raw;
    __device__ __forceinline__ static raw load(const float* p) {
        return *reinterpret_cast<const u32x4*>(p);
    }
    __device__ __forceinline__ static f32x4 get(raw r) { return __builtin_bit_cast(f32x4, r); }
};

// Fragment order ("F-order") of an R x D matrix X (R a multiple of 16, D of
// KG): 16-byte groups, group (rt, sg) holding for lane l the VE elements
// X[16 rt + l%16][KG sg + col(l, e)], e < VE, at element offset
// ((rt * D/KG + sg) * 64 + l) * VE.  A bf16 group is exactly the MFMA A
// fragment of rows 16rt.. and k = 32sg.. (or the B fragment of X^T); an fp32
// group packs the fragments of 4 consecutive k-steps (element e is k-step
// 4sg + e).  Loading one fragment is then one coalesced 16-byte load per lane.
template <typename T> struct FragOrder;
template <> struct FragOrder<bf16> {
    static constexpr int VE = 8, KG = 32;
    __device__ __forceinline__ static int col(int l, int e) { return 8 * (l >> 4) + e; }
    __device__ __forceinline__ static int64_t off(int r, int d, int D) {
        const int dd = d & 31;
        return ((int64_t)(((r >> 4) * (D >> 5) + (d >> 5)) * 64 + (r & 15) + 16 * (dd >> 3)) << 3) +
               (dd & 7);
    }
    __device__ __forceinline__ static Mma<bf16>::frag frag(u32x4 g, int) {
        return __builtin_bit_cast(bf16x8, g);
    }
};
template <> struct FragOrder<float> {
    static constexpr int VE = 4, KG = 16;
    __device__ __forceinline__ static int col(int l, int e) { return 4 * e + (l >> 4); }
    __device__ __forceinline__ static int64_t off(int r, int d, int D) {
        const int dd = d & 15;
        return ((int64_t)(((r >> 4) * (D >> 4) + (d >> 4)) * 64 + (r & 15) + 16 * (dd & 3)) << 2) +
               (dd >> 2);
    }
    __device__ __forceinline__ static Mma<float>::frag frag(u32x4 g, int i) {
        return __uint_as_float(g[i]);
    }
};

// Accumulator order ("C-order") of an R x D matrix: tile (rt, ct) of 64 lanes
// x 4 elements, lane l holding X[16 rt + 4(l/16) + e][16 ct + l%16], the
// layout of an MFMA result tile.  Offset of X[r][d] in elements:
__device__ __forceinline__ int64_t acc_order_off(int r, int d, int D) {
    return ((int64_t)(((r >> 4) * (D >> 4) + (d >> 4)) * 64 + (d & 15) + 16 * ((r & 15) >> 2))
            << 2) + (r & 3);
}

// C(16x16) += A(16 x kn) * B(kn x 16); A row-major at `a` (pitch lda), B
// stored transposed (n-major, k contiguous) at `bt` (pitch ldb).  Pointers
// are tile origins; kn is a multiple of Mma<T>::KSTEP.
template <typename T>
__device__ __forceinline__ f32x4 mma_tile(const T* a, int lda, const T* bt, int ldb, int kn,
                                          int lane, f32x4 c) {
    const T* ar = a + (lane & 15) * lda;
    const T* br = bt + (lane & 15) * ldb;
    for (int k0 = 0; k0 < kn; k0 += Mma<T>::KSTEP)
        c = Mma<T>::mma(Mma<T>::load(ar + k0, lane), Mma<T>::load(br + k0, lane), c);
    return c;
}

// fp32 C(16x16) += A(16 x kn) * B(kn x 16) with both A and B row-major
// (scalar fp32 fragments can be gathered from either layout).
__device__ __forceinline__ f32x4 mma_f32_rr(const float* a, int lda, const float* b, int ldb,
                                            int kn, int lane, f32x4 c) {
    const int r = lane & 15, kk = lane >> 4;
    for (int k0 = 0; k0 < kn; k0 += 4)
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r * lda + k0 + kk], b[(k0 + kk) * ldb + r], c,
                                                 0, 0, 0);
    return c;
}

// Store element e (0..3) of a 16x16 accumulator: row 4*(l/16)+e, col l%16.
__device__ __forceinline__ int acc_row(int lane, int e) { return 4 * (lane >> 4) + e; }
__device__ __forceinline__ int acc_col(int lane) { return lane & 15; }

// Write a 16x16 fp32 accumulator transposed into an n-major T buffer:
// dst[col * ld + row].  The 4 rows a lane holds are consecutive, so this is
// one 8-byte (bf16) or 16-byte (f32) LDS store per lane.
__device__ __forceinline__ void store_acc_t(bf16* dst, int ld, int lane, f32x4 v) {
    uint2 w;
    w.x = pack_bf16x2(v[0], v[1]);
    w.y = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<uint2*>(dst + acc_col(lane) * ld + 4 * (lane >> 4)) = w;
}
__device__ __forceinline__ void store_acc_t(float* dst, int ld, int lane, f32x4 v) {
    *reinterpret_cast<float4*>(dst + acc_col(lane) * ld + 4 * (lane >> 4)) =
        make_float4(v[0], v[1], v[2], v[3]);
}
// The 4 values a lane holds in a tile of X^T are 4 consecutive columns of
// one row of X: store them as one 8-byte (bf16) or 16-byte (f32) write.
__device__ __forceinline__ void store4(bf16* dst, f32x4 v) {
    uint2 w;
    w.x = pack_bf16x2(v[0], v[1]);
    w.y = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<uint2*>(dst) = w;
}
__device__ __forceinline__ void store4(float* dst, f32x4 v) {
    *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
}
// 4 consecutive columns d0..d0+3 (d0 % 4 == 0) of row r of an F-order
// matrix with D columns: one 8-byte store for bf16, four element stores for
// fp32 (whose consecutive columns sit in different lanes' groups).
__device__ __forceinline__ void store4_frag(bf16* base, int r, int d0, int D, f32x4 v) {
    store4(base + FragOrder<bf16>::off(r, d0, D), v);
}
__device__ __forceinline__ void store4_frag(float* base, int r, int d0, int D, f32x4 v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) base[FragOrder<float>::off(r, d0 + e, D)] = v[e];
}
// ... and row-major: dst[row * ld + col] (element stores)
template <typename T>
__device__ __forceinline__ void store_acc(T* dst, int ld, int lane, f32x4 v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) Elem<T>::store(dst + acc_row(lane, e) * ld + acc_col(lane), v[e]);
}

// Copy a rows x cols tile between two row-major buffers with 16-byte vectors.
// cols * sizeof(T) must be a multiple of 16; pitches are in elements.
template <typename T>
__device__ __forceinline__ void copy_tile(T* dst, int64_t ldd, const T* src, int64_t lds, int rows,
                                          int cols, int tid, int nthreads) {
    constexpr int EV = 16 / sizeof(T);
    const int vpr = cols / EV;
    for (int i = tid; i < rows * vpr; i += nthreads) {
        const int r = i / vpr, cv = i - r * vpr;
        *reinterpret_cast<uint4*>(dst + r * ldd + cv * EV) =
            *reinterpret_cast<const uint4*>(src + r * lds + cv * EV);
    }
}

// Wave-wide inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ float wave_incl_scan(float x, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// Sum over the 16 lanes of each DPP row (lanes 16g .. 16g+15) of each of the
// 4 values a lane holds: an inclusive scan by row shifts, whose total lands
// in the row's last lane (l % 16 == 15).
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ f32x4 row_sum16(f32x4 v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float x = v[e];
        x = dpp_add<0x111>(x);   // row_shr:1
        x = dpp_add<0x112>(x);   // row_shr:2
        x = dpp_add<0x114>(x);   // row_shr:4
        x = dpp_add<0x118>(x);   // row_shr:8
        v[e] = x;
    }
    return v;
}
// Sum over the 4 lanes l % 16 == c of one value each (valid in every lane).
__device__ __forceinline__ float sum_groups(float x) {
    x += __shfl_xor(x, 16, 64);
    x += __shfl_xor(x, 32, 64);
    return x;
}

// Store an R x D matrix X, of which an LDS buffer holds the VT columns
// v0 .. v0+VT transposed (X^T rows, pitch ld elements), as fragment-order
// groups of rows 16 rt0 .. 16 (rt0 + nrt) - 1: one 16-byte group per lane,
// each group 1 KB contiguous in HBM.  The transposing LDS reads are those of
// Mma::load_t (bf16) or four element reads (fp32).
template <typename T, int VT>
__device__ __forceinline__ void store_frag_groups(const T* xt, int ld, T* dst, int D, int v0,
                                                  int rt0, int nrt, int lane) {
    typedef FragOrder<T> F;
    constexpr int KG = F::KG, VE = F::VE;
    if constexpr (sizeof(T) == 2 && VT == 16) {
        // half of each 32-column group: lane 16g+n of the group holds columns
        // 8g..8g+7, so the lanes of g = 2hv, 2hv+1 (hv = which half v0 is)
        // store; the others read rows 0..15 of the buffer too (the
        // transposing read addresses rows 8(g%2)..) and drop them
        const int g = lane >> 4, j = lane & 15, hv = (v0 >> 4) & 1;
        typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;
        for (int rt = rt0; rt < rt0 + nrt; ++rt) {
            const T* p = xt + (8 * (g & 1) + (j >> 2)) * ld + 16 * rt + 4 * (j & 3);
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p);
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p + 4 * ld));
            typedef short i16x8 __attribute__((ext_vector_type(8)));
            const u32x4 grp = __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            if ((g >> 1) == hv) {
                const int sg = v0 / KG;
                *reinterpret_cast<u32x4*>(dst + ((int64_t)(rt * (D / KG) + sg) * 64 + lane) * VE) = grp;
            }
        }
        return;
    }
    static_assert(VT % KG == 0 || (sizeof(T) == 2 && VT == 16), "whole or half groups");
    for (int rt = rt0; rt < rt0 + nrt; ++rt) {
#pragma unroll
        for (int q = 0; q < VT / KG; ++q) {
            u32x4 g;
            if constexpr (sizeof(T) == 2) {
                g = __builtin_bit_cast(u32x4, Mma<T>::load_t(xt + KG * q * ld + 16 * rt, ld, lane));
            } else {
#pragma unroll
                for (int e = 0; e < VE; ++e)
                    g[e] = __float_as_uint(xt[(KG * q + F::col(lane, e)) * ld + 16 * rt + (lane & 15)]);
            }
            const int sg = v0 / KG + q;
            *reinterpret_cast<u32x4*>(dst + ((int64_t)(rt * (D / KG) + sg) * 64 + lane) * VE) = g;
        }
    }
}

// Workgroup barrier for LDS hand-offs only: this wave's LDS traffic is done
// (lgkmcnt(0)), then s_barrier.  Unlike __syncthreads() it does not wait for
// the wave's global loads and stores (vmcnt), so loads issued ahead stay in
// flight across it.  Only for kernels whose waves exchange data through LDS
// alone.  The empty asm statements keep the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt not waited for
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
// Wait for this wave's global loads and stores (before it ends with loads in
// flight into registers it no longer reads).
__device__ __forceinline__ void drain_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Run one role of a serial chunk walk over its nch >= 1 steps (every wave
// of the workgroup walks the same number of steps).  The PD+1 register
// buffers rotate with the unrolled steps so each keeps a fixed register set:
// R::step(j, cur, spare) consumes cur and loads step j+PD into spare.
template <int PD, typename R>
__device__ __forceinline__ void drive(R& r, int nch) {
    typename R::Pre b[PD + 1];
#pragma unroll
    for (int q = 0; q < PD; ++q) r.issue(b[q], q);
    lds_barrier();   // the initial carried value is published
    int j = 0;
    for (; j + PD + 1 <= nch; j += PD + 1) {
#pragma unroll
        for (int q = 0; q <= PD; ++q) r.step(j + q, b[q], b[(q + PD) % (PD + 1)]);
    }
#pragma unroll
    for (int q = 0; q < PD; ++q)
        if (j + q < nch) r.step(j + q, b[q], b[(q + PD) % (PD + 1)]);
}

constexpr float LOG2E = 1.4426950408889634f;

// Input activations ("Gated Delta Network（GDN）" §3.1 eq. 5): the natural-log
// gate -exp(A_log) softplus(a + dt_bias) from a raw gate logit a, and beta as
// sigmoid(b) (times 2 for beta in (0, 2)) from a raw logit b.
__device__ __forceinline__ float softplus_f(float x) { return fmaxf(x, 0.f) + log1pf(expf(-fabsf(x))); }
__device__ __forceinline__ float act_log_gate(float a, float A_log, float dt_bias) {
    return -expf(A_log) * softplus_f(a + dt_bias);
}
__device__ __forceinline__ float act_beta(float b, bool neg_eig) {
    const float s = 1.f / (1.f + expf(-b));
    return neg_eig ? 2.f * s : s;
}

// q/k L2 normalisation per token and head ("TileLang 实战" §1.2: unit-norm
// keys keep the write's eigenvalues in [-1, 1]): x / sqrt(sum x^2 + 1e-6),
// the epsilon being this library's reading.  Rows are held as 16-byte pieces
// of T by LPR consecutive lanes (a power of two dividing 64, all 64 lanes
// active); every lane gets its piece scaled by its row's factor.
constexpr float L2_EPS = 1e-6f;
template <typename T, int LPR>
__device__ __forceinline__ u32x4 l2norm_piece(u32x4 p) {
    constexpr int N = 16 / sizeof(T);
    float x[N];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if constexpr (sizeof(T) == 2) {
            x[2 * e] = __uint_as_float(p[e] << 16);
            x[2 * e + 1] = __uint_as_float(p[e] & 0xffff0000u);
        } else {
            x[e] = __uint_as_float(p[e]);
        }
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < N; ++e) ss += x[e] * x[e];
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) ss += __shfl_xor(ss, off, 64);
    const float inv = 1.f / sqrtf(ss + L2_EPS);
    u32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if constexpr (sizeof(T) == 2)
            r[e] = pack_bf16x2(x[2 * e] * inv, x[2 * e + 1] * inv);
        else
            r[e] = __float_as_uint(x[e] * inv);
    }
    return r;
}

}  // namespace gdn
