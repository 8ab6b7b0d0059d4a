// Packed variable-length input: turn the caller's cu_seqlens into the chunk
// table the two prefill stages walk, without a host round trip.
//
// Chunks restart at every sequence start and the last chunk of a sequence is
// ragged ("Gated Delta Network（GDN）", terminology note: a chunk boundary is
// not a sequence boundary; "阅读笔记：DeltaNet 在 FLA 中的代码实现笔记",
// signature of the forward entry: cu_seqlens / chunk_indices).
//
// One workgroup.  Offsets are clamped into [0, T] (end >= start), so invalid
// offsets can give wrong results but never an out-of-bounds access.
//   seqs[n]  = (first token, length, first chunk, order[n])
//   table[c] = (first token, token count, sequence, 0); unused rows have count 0
//   the int32 after seqs[N-1]: 0 if the offsets start at 0, never decrease
//   and end at T, else 1
// order[r] is the sequence of rank r by length, longest first (ties by
// index): the kernels that walk one sequence's chunks serially take their
// workgroups longest first, so the longest chain starts with the first wave
// of workgroups instead of after the short ones (for up to ORDER_MAX
// sequences; beyond that order[r] = r).
// (the table is skipped when its pointer is null: the fused forward needs only seqs)
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

constexpr int ORDER_MAX = 1024;

__global__ __launch_bounds__(256) void table_kernel(TableLaunch a) {
    __shared__ int64_t s_part[256];
    __shared__ int64_t s_carry;
    __shared__ int s_len[ORDER_MAX];
    __shared__ int s_bad;
    const int tid = threadIdx.x;
    if (tid == 0) {
        s_carry = 0;
        s_bad = 0;
    }
    __syncthreads();
    for (int64_t base = 0; base < a.N; base += 256) {
        const int64_t n = base + tid;
        int64_t s = 0, len = 0, nc = 0;
        if (n < a.N) {
            const int64_t rs = a.cu_seqlens[n], re = a.cu_seqlens[n + 1];
            if (re < rs || (n == 0 && rs != 0) || (n == a.N - 1 && re != a.T)) atomicOr(&s_bad, 1);
            s = min(max(rs, (int64_t)0), a.T);
            const int64_t e = min(max(re, s), a.T);
            len = e - s;
            nc = (len + a.C - 1) / a.C;
        }
        s_part[tid] = nc;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {          // inclusive scan
            const int64_t y = tid >= off ? s_part[tid - off] : 0;
            __syncthreads();
            s_part[tid] += y;
            __syncthreads();
        }
        const int64_t first = s_carry + s_part[tid] - nc;
        if (n < a.N) {
            a.seqs[n] = make_int4((int)s, (int)len, (int)min(first, a.max_chunks), (int)n);
            if (a.N <= ORDER_MAX) s_len[n] = (int)len;
            for (int64_t j = 0; a.table && j < nc; ++j) {
                const int64_t c = first + j;
                if (c >= a.max_chunks) break;
                a.table[c] = make_int4((int)(s + j * a.C), (int)min((int64_t)a.C, len - j * a.C),
                                       (int)n, 0);
            }
        }
        __syncthreads();
        if (tid == 255) s_carry += s_part[255];
        __syncthreads();
    }
    if (a.table)
        for (int64_t c = s_carry + tid; c < a.max_chunks; c += 256)
            a.table[c] = make_int4(0, 0, -1, 0);
    __syncthreads();   // every thread's offset check is in s_bad
    if (tid == 0) *reinterpret_cast<int*>(a.seqs + a.N) = s_bad;
    if (a.N <= ORDER_MAX) {   // rank by length: order[rank(n)] = n
        __syncthreads();      // s_len complete, and the identity orders written above
        const int N = (int)a.N;
        for (int n = tid; n < N; n += 256) {
            const int ln = s_len[n];
            int rank = 0;
            for (int m = 0; m < N; ++m) {
                const int lm = s_len[m];
                rank += (lm > ln || (lm == ln && m < n)) ? 1 : 0;
            }
            a.seqs[rank].w = n;
        }
    }
}

hipError_t launch_table(const TableLaunch& a) {
    hipLaunchKernelGGL(table_kernel, dim3(1), dim3(256), 0, a.stream, a);
    return hipGetLastError();
}

}  // namespace gdn
