// Internal launcher interface between the host API (gdn_api.hip) and the
// kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

// In-kernel input activation (the same bits as GDN_ACT_* in gdn.h): the gate
// and beta inputs hold raw logits ("Gated Delta Network（GDN）" §3.1 eq. 5,
// §5 gate fusion); with ACT_QK_L2NORM q and k are L2-normalised per token
// and head as they are read.
enum { ACT_GATE = 1, ACT_BETA_SIGMOID = 2, ACT_BETA_NEG_EIG = 4, ACT_QK_L2NORM = 8 };
struct Act {
    int flags = 0;
    const float* A_log = nullptr;     // [H]
    const float* dt_bias = nullptr;   // [H] (scalar gate) or [H][K] (per-key gate)
};

struct StepLaunch {
    Act act;
    int64_t Hq = 0;         // q/k heads (value heads H are a multiple of it)
    const void *q, *k, *v;
    const float *beta, *g;
    float* state;
    void* o;
    float scale;
    int64_t N, H;
    int K, V;
    bool bf16, per_key;
    hipStream_t stream;
};

// Chunk bookkeeping shared by the two prefill stages.  Without packed
// offsets, chunk c of sequence b covers tokens b*T + j*C .. (j = c % nt).
// With packed offsets a device-built table gives (first token, count, seq).
struct ChunkMap {
    const int4* table;      // [max_chunks] (t0, n, seq, 0) or nullptr
    const int4* seqs;       // [N] (t0, len, first chunk, order[n]: the sequence of
                            // rank n by length, longest first) or nullptr
    int64_t T;              // tokens per sequence when table == nullptr
    int64_t nt;             // chunks per sequence when table == nullptr
    int64_t max_chunks;     // rows of every per-chunk workspace array
};

// Per-chunk intermediates in the workspace, head-major: array[h][chunk][...].
struct ChunkWs {
    float* gcum;   // [H][mc][C] or [H][mc][C][K]   cumulative log2 gate
    void* w;       // [H][mc][C][K]
    void* u;       // [H][mc][C][V]
    void* qs;      // [H][mc][C][K]   scale * Q * gamma
    void* ks;      // [H][mc][C][K]   diag(gamma_C / gamma) K
    void* aqk;     // [H][mc][C][C]
    float* ainv;   // [H][mc][C][C] or nullptr (fp32; the element type in backward mode)
    // backward mode of the intra stage: qs and aqk then hold Qs^T [K][C] and
    // Aqk^T [C][C] in fragment order, and these two are written as well
    void* ksr = nullptr;   // [H][mc][C][K]   Ks in fragment order (rows = tokens)
    void* wt = nullptr;    // [H][mc][K][C]   W^T in fragment order
};

struct IntraLaunch {
    Act act;
    int64_t Hq = 0;         // q/k heads (value heads H are a multiple of it)
    const void *q, *k, *v;
    const float *beta, *g;
    ChunkMap map;
    ChunkWs ws;
    int64_t H;
    int K, V, C;
    float scale;
    bool bf16, per_key;
    bool bwd = false;       // write the backward operand orders (and the whole per-key gate)
    hipStream_t stream;
};

struct ScanLaunch {
    ChunkMap map;
    ChunkWs ws;
    const float* h0;
    float* ht;
    void* o;                // nullptr: the output is not computed
    void* hs = nullptr;     // [H][mc][K x V] state entering each chunk (fragment order), or nullptr
    void* vn = nullptr;     // [H][mc][C x V] V_new of each chunk (fragment order), or nullptr
    int64_t N, H;
    int K, V, C;
    bool bf16, per_key;
    hipStream_t stream;
};

// Backward, reverse state-gradient pass: serial over the chunks of one
// (sequence, head), last chunk first, parallel over value slices.
struct BwdScanLaunch {
    ChunkMap map;
    const float* gcum;      // [H][mc][C] (or [H][mc][C][K]) cumulative log2 gate
    const void* ksr;        // Ks, Aqk^T, Qs^T, W^T per chunk in fragment order
    const void* aqkt;
    const void* qst;
    const void* wt;
    const void* dout;       // [B,T,H,V] output gradient
    const float* dht;       // [N,H,K,V] or nullptr
    float* dh0;             // [N,H,K,V] or nullptr
    void* dhs;              // [H][mc][K x V] gradient of the state leaving each chunk (fragment order)
    void* dvn;              // [H][mc][C x V] gradient of V_new (fragment order)
    int64_t N, H;
    int K, V, C;
    bool bf16;
    bool per_key = false;   // the carried gradient decays row by row
    hipStream_t stream;
};

// Backward, per-chunk gradients: one workgroup per (chunk, head).
struct BwdLocalLaunch {
    ChunkMap map;
    const void *q, *k, *v, *dout;
    const float *beta, *gcum;   // gcum [H][mc][C] or, per-key gate, [H][mc][C][K]
    const void* ainv;       // [H][mc][C][C] (I + A)^{-1}, element type, row-major
    const void *hs, *dhs, *vn, *dvn;
    void *dq, *dk, *dv;
    float *dbeta, *dg;
    // grouped value heads: q/k have Hq heads; value head h reads q/k head
    // h / (H / Hq) and, when H > Hq, leaves its dq, dk terms in these fp32
    // [B*T][H][K] buffers for launch_gva_sum (dq, dk unused then)
    float *dq_part = nullptr, *dk_part = nullptr;
    // input activation: beta and g hold raw logits; dbeta and dg are then the
    // gradients of the logits, and each (head, chunk slot) leaves its sums of
    // dg * log alpha and of d(logit a) in act_part[h][slot][2] (per-key gate:
    // [h][slot][K + 2], the sum of dg * log alpha first, the K per-channel
    // sums from index 2) for launch_act_reduce
    Act act;
    const float* g = nullptr;   // the raw gate logits [B*T][H] (with ACT_GATE)
    float* act_part = nullptr;
    int64_t Hq = 0;
    int64_t H;
    int K, V, C;
    float scale;
    bool bf16;
    bool per_key = false;
    hipStream_t stream;
};

// dA_log[h], ddt_bias[h] (or [h][K]): the sums of the per-chunk terms over the used slots
struct ActReduceLaunch {
    ChunkMap map;
    const float* part;      // [H][max_chunks][2], or [H][max_chunks][K + 2] per-key
    float *dA_log, *ddt_bias;
    int64_t H;
    int K = 0;              // per-key gate: the channels; 0 for the scalar gate
    hipStream_t stream;
};

// dq (dk) of q/k head hq = the sum of the fp32 terms of its H/Hq value heads
struct GvaSumLaunch {
    const float* part;      // [rows][H][K]
    void* out;              // [rows][Hq][K], element type
    int64_t rows, H, Hq;
    int K;
    bool bf16;
    hipStream_t stream;
};

// The fused forward (bf16 q/k/v, scalar gate, K and V each 64 or 128, C = 64):
// one kernel per call, no per-chunk intermediates in HBM.
struct FusedLaunch {
    Act act;
    int64_t Hq = 0;         // q/k heads (value heads H are a multiple of it)
    const void *q, *k, *v;
    const float *beta, *g;
    const float* h0;
    float* ht;
    void* o;
    const int4* seqs;       // [N] (t0, len, ...) for packed input, else nullptr
    int* sync_status;       // set to 1 by a wave whose bounded wait gave up, or nullptr
    bool loads_first = false;   // issue each chunk's loads before its gate arrays
    int64_t T;              // tokens per sequence when seqs == nullptr
    int64_t N, H;
    int K, V, C;
    float scale;
    bool bf16, per_key;
    hipStream_t stream;
};

struct TableLaunch {
    const int64_t* cu_seqlens;
    int64_t N, T;
    int C;
    int4* table;            // nullptr: write only seqs
    int4* seqs;
    int64_t max_chunks;
    hipStream_t stream;
};

hipError_t launch_step(const StepLaunch& a);
hipError_t launch_table(const TableLaunch& a);
hipError_t launch_intra(const IntraLaunch& a);
hipError_t launch_scan(const ScanLaunch& a);
bool fused_supported(const FusedLaunch& a);
hipError_t launch_fused(const FusedLaunch& a);
hipError_t launch_bwd_scan(const BwdScanLaunch& a);
hipError_t launch_bwd_local(const BwdLocalLaunch& a);       // dispatches per_key to the next
hipError_t launch_bwd_local_kda(const BwdLocalLaunch& a);
hipError_t launch_gva_sum(const GvaSumLaunch& a);
hipError_t launch_act_reduce(const ActReduceLaunch& a);

// Chain rule of the q/k L2 normalisation, in place: dx = (dy - x (x.dy) / n2)
// / sqrt(n2) with n2 = sum x^2 + 1e-6 per row of K elements (x raw, dy the
// gradient of the normalised row, both of the element type).
struct L2BwdLaunch {
    const void* x;
    void* dx;               // holds dy on entry
    int64_t rows;
    int K;
    bool bf16;
    hipStream_t stream;
};
hipError_t launch_l2norm_bwd(const L2BwdLaunch& a);

}  // namespace gdn
