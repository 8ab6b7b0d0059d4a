// Host side of the C ABI declared in include/gdn.h: argument checks,
// workspace layout and the kernel launches.  Nothing here allocates memory or
// synchronises; every launch goes to the caller's stream.
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/gdn.h"
#include "gdn_launch.hpp"

namespace {

thread_local char g_err[512];

gdn_status fail(gdn_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
gdn_status fail(gdn_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

gdn_status ok() {
    g_err[0] = 0;
    return GDN_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }
bool aligned8(const void* p) { return ((uintptr_t)p & 7u) == 0; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool dim_ok(int64_t d) { return d == 64 || d == 128; }

// value heads (GVA: a multiple of the q/k heads)
int64_t vheads(const gdn_fwd_desc* d) { return d->num_v_heads > 0 ? d->num_v_heads : d->num_heads; }

gdn_status check_desc(const gdn_fwd_desc* d, bool packed) {
    if (!d) return fail(GDN_ERR_NULL_ARG, "desc is NULL");
    if (d->qkv_dtype != GDN_DTYPE_F32 && d->qkv_dtype != GDN_DTYPE_BF16)
        return fail(GDN_ERR_BAD_DTYPE, "qkv_dtype %d", d->qkv_dtype);
    if (d->gate != GDN_GATE_SCALAR && d->gate != GDN_GATE_PER_KEY)
        return fail(GDN_ERR_BAD_DTYPE, "gate %d", d->gate);
    if (d->batch <= 0 || d->seq_len < 0 || d->num_heads <= 0 || d->key_dim <= 0 ||
        d->value_dim <= 0)
        return fail(GDN_ERR_BAD_SHAPE, "non-positive size (B=%lld T=%lld H=%lld K=%lld V=%lld)",
                    (long long)d->batch, (long long)d->seq_len, (long long)d->num_heads,
                    (long long)d->key_dim, (long long)d->value_dim);
    if (packed && d->batch != 1)
        return fail(GDN_ERR_BAD_SHAPE, "packed sequences need batch == 1 (got %lld)",
                    (long long)d->batch);
    if (packed && d->num_seqs <= 0)
        return fail(GDN_ERR_BAD_SHAPE, "packed sequences need num_seqs > 0");
    if (d->batch * d->seq_len >= (int64_t)1 << 31)
        return fail(GDN_ERR_BAD_SHAPE, "B*T must be below 2^31");
    if (d->num_heads > 65535) return fail(GDN_ERR_BAD_SHAPE, "num_heads above 65535");
    if (d->num_v_heads < 0 || (d->num_v_heads > 0 && (d->num_v_heads % d->num_heads != 0 ||
                                                      d->num_v_heads > 65535)))
        return fail(GDN_ERR_BAD_SHAPE, "num_v_heads %lld must be 0 or a multiple of num_heads %lld",
                    (long long)d->num_v_heads, (long long)d->num_heads);
    if (d->chunk != 64)
        return fail(GDN_ERR_UNSUPPORTED, "chunk %d: only the 64-token tiling is built", d->chunk);
    if (!dim_ok(d->key_dim) || !dim_ok(d->value_dim))
        return fail(GDN_ERR_UNSUPPORTED, "K=%lld V=%lld (supported: 64, 128)",
                    (long long)d->key_dim, (long long)d->value_dim);
    if (d->qkv_dtype == GDN_DTYPE_F32 && d->gate == GDN_GATE_PER_KEY && d->key_dim == 128)
        return fail(GDN_ERR_UNSUPPORTED, "fp32 q/k/v with the per-key gate needs K = 64");
    return GDN_OK;
}

int64_t max_chunks_of(const gdn_fwd_desc* d, bool packed) {
    const int64_t nt = (d->seq_len + d->chunk - 1) / d->chunk;
    return packed ? nt + d->num_seqs : d->batch * nt;
}

void layout(const gdn_fwd_desc* d, bool packed, gdn_workspace_layout* L) {
    const int64_t mc = max_chunks_of(d, packed);
    const int64_t H = vheads(d), K = d->key_dim, V = d->value_dim, C = d->chunk;
    const size_t es = d->qkv_dtype == GDN_DTYPE_BF16 ? 2 : 4;
    const size_t blocks = (size_t)(H * mc);
    size_t off = 0;
    L->gcum = off;
    off = align256(off + blocks * C * (d->gate == GDN_GATE_PER_KEY ? K : 1) * 4);
    L->w = off;
    off = align256(off + blocks * C * K * es);
    L->u = off;
    off = align256(off + blocks * C * V * es);
    L->qs = off;
    off = align256(off + blocks * C * K * es);
    L->ks = off;
    off = align256(off + blocks * C * K * es);
    L->aqk = off;
    off = align256(off + blocks * C * C * es);
    L->ainv = off;
    off = align256(off + blocks * C * C * 4);
    L->chunks = off;
    L->seqs = off + (size_t)mc * 16;
    // (packed: the per-sequence records, then the offsets' check word)
    off = align256(off + (size_t)mc * 16 + (size_t)(packed ? d->num_seqs + 1 : 0) * 16);
    L->total = off;
    L->max_chunks = mc;
}

// Backward workspace: the forward layout (intra stage in backward mode, the
// chunk table), then the extra operand orders, the entry states, V_new and
// the two gradients the reverse pass leaves for the per-chunk kernel.
struct BwdLayout {
    gdn_workspace_layout f;
    size_t ksr, wt, hs, dhs, vn, dvn, dq_part, dk_part, act_part, total;
};

void bwd_layout(const gdn_fwd_desc* d, bool packed, BwdLayout* L) {
    layout(d, packed, &L->f);
    const int64_t mc = L->f.max_chunks;
    const int64_t H = vheads(d), K = d->key_dim, V = d->value_dim, C = d->chunk;
    const size_t es = d->qkv_dtype == GDN_DTYPE_BF16 ? 2 : 4;
    const size_t blocks = (size_t)(H * mc);
    size_t off = L->f.total;
    L->ksr = off;
    off = align256(off + blocks * C * K * es);
    L->wt = off;
    off = align256(off + blocks * C * K * es);
    L->hs = off;
    off = align256(off + blocks * K * V * es);
    L->dhs = off;
    off = align256(off + blocks * K * V * es);
    L->vn = off;
    off = align256(off + blocks * C * V * es);
    L->dvn = off;
    off = align256(off + blocks * C * V * es);
    // grouped value heads: each value head's dq, dk terms (fp32) before the
    // sum over the heads that share a q/k head
    const bool gva = H > d->num_heads;
    const size_t rows = (size_t)(d->batch * d->seq_len);
    L->dq_part = off;
    off = align256(off + (gva ? rows * H * K * 4 : 0));
    L->dk_part = off;
    off = align256(off + (gva ? rows * H * K * 4 : 0));
    // input activation: per (head, chunk slot) terms of dA_log and ddt_bias
    // (per-key gate: ddt_bias per channel)
    L->act_part = off;
    off = align256(off + blocks * (d->gate == GDN_GATE_PER_KEY ? K + 2 : 2) * 4);
    L->total = off;
}

gdn_status check_bwd_desc(const gdn_fwd_desc* d, bool packed) {
    gdn_status s = check_desc(d, packed);
    if (s != GDN_OK) return s;
    if (d->gate == GDN_GATE_PER_KEY && d->qkv_dtype != GDN_DTYPE_BF16)
        return fail(GDN_ERR_UNSUPPORTED, "the per-key gate's backward needs bf16 q/k/v");
    if (d->qkv_dtype == GDN_DTYPE_F32 && (d->key_dim != 64 || d->value_dim != 64))
        return fail(GDN_ERR_UNSUPPORTED, "fp32 backward needs K = V = 64");
    return GDN_OK;
}

// gdn_chunk_fwd runs the fused kernel for these shapes; its workspace holds
// only the per-sequence records of packed input
bool fused_path(const gdn_fwd_desc* d, int act_flags = 0) {
    (void)act_flags;   // every activation runs on either route
    gdn::FusedLaunch f{};
    f.bf16 = d->qkv_dtype == GDN_DTYPE_BF16;
    f.per_key = d->gate == GDN_GATE_PER_KEY;
    f.K = (int)d->key_dim;
    f.V = (int)d->value_dim;
    f.C = d->chunk;
    return gdn::fused_supported(f);
}

// Single-pass workspace: the per-sequence records of packed input and the
// check word of cu_seqlens, then a 256-byte block whose first int32 is the
// synchronisation status word (gdn_sync_status_offset)
size_t fused_sync_offset(const gdn_fwd_desc* d, bool packed) {
    return align256((size_t)(packed ? d->num_seqs + 1 : 1) * 16);
}
size_t fused_workspace(const gdn_fwd_desc* d, bool packed) { return fused_sync_offset(d, packed) + 256; }

gdn_status hip_fail(hipError_t e, const char* what) {
    return fail(GDN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

struct Prepared {
    gdn::ChunkMap map;
    gdn::ChunkWs ws;
};

static_assert(GDN_ACT_GATE == gdn::ACT_GATE && GDN_ACT_BETA_SIGMOID == gdn::ACT_BETA_SIGMOID &&
                  GDN_ACT_BETA_NEG_EIG == gdn::ACT_BETA_NEG_EIG && GDN_ACT_QK_L2NORM == gdn::ACT_QK_L2NORM,
              "activation bits");

// the optional input activation (NULL: g and beta are used as given)
gdn_status check_act(const gdn_activation* act, gdn::Act* out) {
    *out = gdn::Act{};
    if (!act || act->flags == 0) return GDN_OK;
    const int known = GDN_ACT_GATE | GDN_ACT_BETA_SIGMOID | GDN_ACT_BETA_NEG_EIG | GDN_ACT_QK_L2NORM;
    if (act->flags & ~known) return fail(GDN_ERR_UNSUPPORTED, "activation flags 0x%x", act->flags);
    if ((act->flags & GDN_ACT_BETA_NEG_EIG) && !(act->flags & GDN_ACT_BETA_SIGMOID))
        return fail(GDN_ERR_UNSUPPORTED, "GDN_ACT_BETA_NEG_EIG needs GDN_ACT_BETA_SIGMOID");
    if (act->flags & GDN_ACT_GATE) {
        if (!act->A_log || !act->dt_bias)
            return fail(GDN_ERR_NULL_ARG, "GDN_ACT_GATE needs A_log and dt_bias");
        if (!aligned4(act->A_log) || !aligned4(act->dt_bias))
            return fail(GDN_ERR_MISALIGNED, "A_log and dt_bias need 4-byte alignment");
    }
    out->flags = act->flags;
    out->A_log = act->A_log;
    out->dt_bias = act->dt_bias;
    return GDN_OK;
}

gdn_status prepare(const gdn_fwd_desc* d, const void* q, const void* k, const void* v,
                   const float* beta, const float* g, const int64_t* cu_seqlens, void* workspace,
                   size_t workspace_bytes, bool want_ainv, hipStream_t stream, Prepared* P,
                   const gdn::Act& act = gdn::Act{}) {
    const bool packed = cu_seqlens != nullptr;
    gdn_status s = check_desc(d, packed);
    if (s != GDN_OK) return s;
    if (!packed && d->num_seqs != 0)
        return fail(GDN_ERR_BAD_SHAPE, "num_seqs must be 0 without cu_seqlens");
    if (!q || !k || !v || !beta || !g || !workspace)
        return fail(GDN_ERR_NULL_ARG, "q, k, v, beta, g and workspace are required");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned4(beta) || !aligned4(g) ||
        !aligned8(cu_seqlens))
        return fail(GDN_ERR_MISALIGNED,
                    "q, k, v need 16-byte, beta and g 4-byte, cu_seqlens 8-byte alignment");
    if (((uintptr_t)workspace & 255u) != 0)
        return fail(GDN_ERR_MISALIGNED, "workspace must be 256-byte aligned");
    gdn_workspace_layout L;
    layout(d, packed, &L);
    if (workspace_bytes < L.total)
        return fail(GDN_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, need %zu", workspace_bytes,
                    L.total);
    char* ws = static_cast<char*>(workspace);
    P->ws.gcum = reinterpret_cast<float*>(ws + L.gcum);
    P->ws.w = ws + L.w;
    P->ws.u = ws + L.u;
    P->ws.aqk = ws + L.aqk;
    P->ws.ainv = want_ainv ? reinterpret_cast<float*>(ws + L.ainv) : nullptr;
    P->ws.qs = ws + L.qs;
    P->ws.ks = ws + L.ks;
    P->map.max_chunks = L.max_chunks;
    P->map.T = d->seq_len;
    P->map.nt = (d->seq_len + d->chunk - 1) / d->chunk;
    if (packed) {
        P->map.table = reinterpret_cast<const int4*>(ws + L.chunks);
        P->map.seqs = reinterpret_cast<const int4*>(ws + L.seqs);
        gdn::TableLaunch t;
        t.cu_seqlens = cu_seqlens;
        t.N = d->num_seqs;
        t.T = d->seq_len;
        t.C = d->chunk;
        t.table = const_cast<int4*>(P->map.table);
        t.seqs = const_cast<int4*>(P->map.seqs);
        t.max_chunks = L.max_chunks;
        t.stream = stream;
        hipError_t e = gdn::launch_table(t);
        if (e != hipSuccess) return hip_fail(e, "chunk table launch");
    } else {
        P->map.table = nullptr;
        P->map.seqs = nullptr;
    }
    if (L.max_chunks > 0 && d->seq_len > 0) {
        gdn::IntraLaunch a;
        a.q = q;
        a.k = k;
        a.v = v;
        a.beta = beta;
        a.g = g;
        a.map = P->map;
        a.ws = P->ws;
        a.H = vheads(d);
        a.Hq = d->num_heads;
        a.K = (int)d->key_dim;
        a.V = (int)d->value_dim;
        a.C = d->chunk;
        a.scale = d->scale;
        a.bf16 = d->qkv_dtype == GDN_DTYPE_BF16;
        a.per_key = d->gate == GDN_GATE_PER_KEY;
        a.act = act;
        a.stream = stream;
        hipError_t e = gdn::launch_intra(a);
        if (e != hipSuccess) return hip_fail(e, "intra-chunk launch");
    }
    return GDN_OK;
}

// ---- the allocation-free variant of the single-pass forward
// Its scratch (the per-sequence records of packed input and the check word
// of cu_seqlens) lives in this file-scope device array: each GPU the library
// runs on holds its own copy until the process ends.  Host code never uses
// the array's name as an address: the address of the current device's copy
// comes from hipGetSymbolAddress, once per device.
constexpr int64_t NOALLOC_MAX_SEQS = GDN_NOALLOC_MAX_SEQS;
constexpr size_t NOALLOC_BYTES = ((NOALLOC_MAX_SEQS + 1) * 16 + 255) / 256 * 256 + 256;
static __device__ __align__(256) unsigned char scratch[NOALLOC_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch[MAX_DEVICES] = {};

gdn_status scratch_of_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= MAX_DEVICES) return fail(GDN_ERR_UNSUPPORTED, "device %d", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(GDN_ERR_HIP, "hipGetSymbolAddress(scratch) gave a null address");
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return GDN_OK;
}

}  // namespace

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char* gdn_status_str(gdn_status s) {
    switch (s) {
        case GDN_OK: return "GDN_OK";
        case GDN_ERR_NULL_ARG: return "GDN_ERR_NULL_ARG";
        case GDN_ERR_BAD_SHAPE: return "GDN_ERR_BAD_SHAPE";
        case GDN_ERR_BAD_DTYPE: return "GDN_ERR_BAD_DTYPE";
        case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED";
        case GDN_ERR_WORKSPACE_TOO_SMALL: return "GDN_ERR_WORKSPACE_TOO_SMALL";
        case GDN_ERR_MISALIGNED: return "GDN_ERR_MISALIGNED";
        case GDN_ERR_HIP: return "GDN_ERR_HIP";
        case GDN_ERR_BAD_SEQLENS: return "GDN_ERR_BAD_SEQLENS";
        default: return "GDN_ERR_UNKNOWN";
    }
}

const char* gdn_last_error(void) { return g_err; }

gdn_status gdn_workspace_layout_of(const gdn_fwd_desc* d, gdn_workspace_layout* out) {
    if (!out) return fail(GDN_ERR_NULL_ARG, "out is NULL");
    const bool packed = d && d->num_seqs > 0;
    gdn_status s = check_desc(d, packed);
    if (s != GDN_OK) return s;
    layout(d, packed, out);
    return ok();
}

gdn_status gdn_chunk_fwd_workspace_act(const gdn_fwd_desc* d, const gdn_activation* act_in,
                                       size_t* bytes) {
    if (!bytes) return fail(GDN_ERR_NULL_ARG, "bytes is NULL");
    gdn::Act act;
    gdn_status s = check_act(act_in, &act);
    if (s != GDN_OK) return s;
    gdn_workspace_layout L;
    s = gdn_workspace_layout_of(d, &L);
    if (s != GDN_OK) return s;
    *bytes = fused_path(d, act.flags) ? fused_workspace(d, d->num_seqs > 0) : L.total;
    return ok();
}

gdn_status gdn_seqlens_status_offset(const gdn_fwd_desc* d, const gdn_activation* act_in,
                                     int32_t backward, size_t* offset) {
    if (!offset) return fail(GDN_ERR_NULL_ARG, "offset is NULL");
    gdn_status s = backward ? check_bwd_desc(d, true) : check_desc(d, true);
    if (s != GDN_OK) return s;
    gdn::Act act;
    s = check_act(act_in, &act);
    if (s != GDN_OK) return s;
    // the word follows the num_seqs 16-byte records of the sequence table
    const size_t rec = (size_t)d->num_seqs * 16;
    if (backward) {
        BwdLayout L;
        bwd_layout(d, true, &L);
        *offset = L.f.seqs + rec;
    } else if (fused_path(d, act.flags)) {
        *offset = rec;
    } else {
        gdn_workspace_layout L;
        layout(d, true, &L);
        *offset = L.seqs + rec;
    }
    return ok();
}

gdn_status gdn_sync_status_offset(const gdn_fwd_desc* d, const gdn_activation* act_in,
                                  size_t* offset) {
    if (!offset) return fail(GDN_ERR_NULL_ARG, "offset is NULL");
    const bool packed = d && d->num_seqs > 0;
    gdn_status s = check_desc(d, packed);
    if (s != GDN_OK) return s;
    gdn::Act act;
    s = check_act(act_in, &act);
    if (s != GDN_OK) return s;
    if (!fused_path(d, act.flags))
        return fail(GDN_ERR_UNSUPPORTED, "this shape runs the two-stage route, which has no waits");
    *offset = fused_sync_offset(d, packed);
    return ok();
}

gdn_status gdn_chunk_fwd_workspace(const gdn_fwd_desc* d, size_t* bytes) {
    return gdn_chunk_fwd_workspace_act(d, nullptr, bytes);
}

gdn_status gdn_chunk_intra(const gdn_fwd_desc* d, const void* q, const void* k, const void* v,
                           const float* beta, const float* g, const int64_t* cu_seqlens,
                           void* workspace, size_t workspace_bytes, int32_t flags, void* stream) {
    Prepared P;
    gdn_status s = prepare(d, q, k, v, beta, g, cu_seqlens, workspace, workspace_bytes,
                           (flags & GDN_INTRA_STORE_AINV) != 0, static_cast<hipStream_t>(stream),
                           &P);
    return s == GDN_OK ? ok() : s;
}

static gdn_status scan(const gdn_fwd_desc* d, const float* h0, const int64_t* cu_seqlens,
                       void* o, float* ht, void* workspace, size_t workspace_bytes,
                       hipStream_t st) {
    const bool packed = cu_seqlens != nullptr;
    gdn_status s = check_desc(d, packed);
    if (s != GDN_OK) return s;
    if (!o || !workspace) return fail(GDN_ERR_NULL_ARG, "o and workspace are required");
    if (!aligned16(o) || !aligned4(h0) || !aligned4(ht))
        return fail(GDN_ERR_MISALIGNED, "o needs 16-byte, h0 and ht 4-byte alignment");
    if (((uintptr_t)workspace & 255u) != 0)
        return fail(GDN_ERR_MISALIGNED, "workspace must be 256-byte aligned");
    gdn_workspace_layout L;
    layout(d, packed, &L);
    if (workspace_bytes < L.total)
        return fail(GDN_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, need %zu", workspace_bytes,
                    L.total);
    char* ws = static_cast<char*>(workspace);
    gdn::ScanLaunch a;
    a.map.max_chunks = L.max_chunks;
    a.map.T = d->seq_len;
    a.map.nt = (d->seq_len + d->chunk - 1) / d->chunk;
    a.map.table = packed ? reinterpret_cast<const int4*>(ws + L.chunks) : nullptr;
    a.map.seqs = packed ? reinterpret_cast<const int4*>(ws + L.seqs) : nullptr;
    a.ws.gcum = reinterpret_cast<float*>(ws + L.gcum);
    a.ws.w = ws + L.w;
    a.ws.u = ws + L.u;
    a.ws.qs = ws + L.qs;
    a.ws.ks = ws + L.ks;
    a.ws.aqk = ws + L.aqk;
    a.ws.ainv = nullptr;
    a.h0 = h0;
    a.ht = ht;
    a.o = o;
    a.N = packed ? d->num_seqs : d->batch;
    a.H = vheads(d);
    a.K = (int)d->key_dim;
    a.V = (int)d->value_dim;
    a.C = d->chunk;
    a.bf16 = d->qkv_dtype == GDN_DTYPE_BF16;
    a.per_key = d->gate == GDN_GATE_PER_KEY;
    a.stream = st;
    hipError_t e = gdn::launch_scan(a);
    if (e != hipSuccess) return hip_fail(e, "state pass launch");
    return ok();
}

gdn_status gdn_chunk_scan(const gdn_fwd_desc* d, const float* h0, const int64_t* cu_seqlens,
                          void* o, float* ht, void* workspace, size_t workspace_bytes,
                          void* stream) {
    return scan(d, h0, cu_seqlens, o, ht, workspace, workspace_bytes,
                static_cast<hipStream_t>(stream));
}

static gdn_status fused_fwd(const gdn_fwd_desc* d, const void* q, const void* k, const void* v,
                            const float* beta, const float* g, const float* h0,
                            const int64_t* cu_seqlens, void* o, float* ht, void* workspace,
                            size_t workspace_bytes, hipStream_t st, const gdn::Act& act,
                            bool report_sync = true) {
    const bool packed = cu_seqlens != nullptr;
    if (!packed && d->num_seqs != 0)
        return fail(GDN_ERR_BAD_SHAPE, "num_seqs must be 0 without cu_seqlens");
    if (!q || !k || !v || !beta || !g || !workspace)
        return fail(GDN_ERR_NULL_ARG, "q, k, v, beta, g and workspace are required");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned4(beta) || !aligned4(g) ||
        !aligned8(cu_seqlens))
        return fail(GDN_ERR_MISALIGNED,
                    "q, k, v need 16-byte, beta and g 4-byte, cu_seqlens 8-byte alignment");
    if (((uintptr_t)workspace & 255u) != 0)
        return fail(GDN_ERR_MISALIGNED, "workspace must be 256-byte aligned");
    const size_t need = fused_workspace(d, packed);
    if (workspace_bytes < need)
        return fail(GDN_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, need %zu", workspace_bytes,
                    need);
    gdn::FusedLaunch a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.beta = beta;
    a.g = g;
    a.h0 = h0;
    a.ht = ht;
    a.o = o;
    a.seqs = nullptr;
    a.sync_status = report_sync ? reinterpret_cast<int*>(static_cast<char*>(workspace) +
                                                         fused_sync_offset(d, packed))
                                : nullptr;
    a.T = d->seq_len;
    a.N = packed ? d->num_seqs : d->batch;
    a.H = vheads(d);
    a.Hq = d->num_heads;
    {   // inputs beyond the 256 MB Infinity Cache are read from HBM
        const double tokens = (double)d->batch * (double)d->seq_len;
        const double in_bytes = tokens * ((double)(2 * d->num_heads * d->key_dim) * 2 +
                                          (double)(a.H * d->value_dim) * 2 + (double)a.H * 8);
        a.loads_first = in_bytes > (double)(256u << 20);
    }
    a.K = (int)d->key_dim;
    a.V = (int)d->value_dim;
    a.C = d->chunk;
    a.scale = d->scale;
    a.bf16 = true;
    a.per_key = false;
    a.act = act;
    a.stream = st;
    if (packed) {
        gdn::TableLaunch t;
        t.cu_seqlens = cu_seqlens;
        t.N = d->num_seqs;
        t.T = d->seq_len;
        t.C = d->chunk;
        t.table = nullptr;
        t.seqs = static_cast<int4*>(workspace);
        t.max_chunks = max_chunks_of(d, true);
        t.stream = st;
        hipError_t e = gdn::launch_table(t);
        if (e != hipSuccess) return hip_fail(e, "sequence table launch");
        a.seqs = static_cast<const int4*>(workspace);
    }
    hipError_t e = gdn::launch_fused(a);
    if (e != hipSuccess) return hip_fail(e, "fused forward launch");
    return ok();
}

gdn_status gdn_chunk_fwd_act(const gdn_fwd_desc* d, const gdn_activation* act_in, const void* q,
                             const void* k, const void* v, const float* beta, const float* g,
                             const float* h0, const int64_t* cu_seqlens, void* o, float* ht,
                             void* workspace, size_t workspace_bytes, void* stream) {
    const bool packed = cu_seqlens != nullptr;
    gdn_status s = check_desc(d, packed);
    if (s != GDN_OK) return s;
    gdn::Act act;
    s = check_act(act_in, &act);
    if (s != GDN_OK) return s;
    if (!o) return fail(GDN_ERR_NULL_ARG, "o is NULL");
    if (!aligned16(o) || !aligned4(h0) || !aligned4(ht))
        return fail(GDN_ERR_MISALIGNED, "o needs 16-byte, h0 and ht 4-byte alignment");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (fused_path(d, act.flags)) return fused_fwd(d, q, k, v, beta, g, h0, cu_seqlens, o, ht, workspace,
                                        workspace_bytes, st, act);
    Prepared P;
    s = prepare(d, q, k, v, beta, g, cu_seqlens, workspace, workspace_bytes, false, st, &P, act);
    if (s != GDN_OK) return s;
    return scan(d, h0, cu_seqlens, o, ht, workspace, workspace_bytes, st);
}

gdn_status gdn_chunk_fwd_noalloc(const gdn_fwd_desc* d, const gdn_activation* act_in,
                                 const void* q, const void* k, const void* v, const float* beta,
                                 const float* g, const float* h0, const int64_t* cu_seqlens,
                                 void* o, float* ht, void* stream) {
    const bool packed = cu_seqlens != nullptr;
    gdn_status s = check_desc(d, packed);
    if (s != GDN_OK) return s;
    gdn::Act act;
    s = check_act(act_in, &act);
    if (s != GDN_OK) return s;
    if (!fused_path(d, act.flags))
        return fail(GDN_ERR_UNSUPPORTED,
                    "gdn_chunk_fwd_noalloc runs the single-pass kernel only (bf16 q/k/v, scalar "
                    "gate, K and V each 64 or 128, chunk 64)");
    if (packed && d->num_seqs > NOALLOC_MAX_SEQS)
        return fail(GDN_ERR_UNSUPPORTED, "gdn_chunk_fwd_noalloc takes at most %lld packed sequences "
                    "(got %lld)", (long long)NOALLOC_MAX_SEQS, (long long)d->num_seqs);
    if (!o) return fail(GDN_ERR_NULL_ARG, "o is NULL");
    if (!aligned16(o) || !aligned4(h0) || !aligned4(ht))
        return fail(GDN_ERR_MISALIGNED, "o needs 16-byte, h0 and ht 4-byte alignment");
    if (fused_workspace(d, packed) > NOALLOC_BYTES)
        return fail(GDN_ERR_UNSUPPORTED, "scratch of %zu bytes exceeds the library's %zu",
                    fused_workspace(d, packed), NOALLOC_BYTES);
    void* ws = nullptr;
    s = scratch_of_current_device(&ws);
    if (s != GDN_OK) return s;
    return fused_fwd(d, q, k, v, beta, g, h0, cu_seqlens, o, ht, ws, NOALLOC_BYTES,
                     static_cast<hipStream_t>(stream), act, /*report_sync=*/false);
}

gdn_status gdn_chunk_fwd(const gdn_fwd_desc* d, const void* q, const void* k, const void* v,
                         const float* beta, const float* g, const float* h0,
                         const int64_t* cu_seqlens, void* o, float* ht, void* workspace,
                         size_t workspace_bytes, void* stream) {
    return gdn_chunk_fwd_act(d, nullptr, q, k, v, beta, g, h0, cu_seqlens, o, ht, workspace,
                             workspace_bytes, stream);
}

gdn_status gdn_chunk_bwd_workspace(const gdn_fwd_desc* d, size_t* bytes) {
    if (!bytes) return fail(GDN_ERR_NULL_ARG, "bytes is NULL");
    const bool packed = d && d->num_seqs > 0;
    gdn_status s = check_bwd_desc(d, packed);
    if (s != GDN_OK) return s;
    BwdLayout L;
    bwd_layout(d, packed, &L);
    *bytes = L.total;
    return ok();
}

gdn_status gdn_chunk_bwd_act(const gdn_fwd_desc* d, const gdn_activation* act_in, const void* q,
                             const void* k, const void* v, const float* beta, const float* g,
                             const float* h0, const int64_t* cu_seqlens, const void* dout,
                             const float* dht, void* dq, void* dk, void* dv, float* dbeta,
                             float* dg, float* dh0, float* dA_log, float* ddt_bias,
                             void* workspace, size_t workspace_bytes, void* stream) {
    const bool packed = cu_seqlens != nullptr;
    gdn_status s = check_bwd_desc(d, packed);
    if (s != GDN_OK) return s;
    gdn::Act act;
    s = check_act(act_in, &act);
    if (s != GDN_OK) return s;
    const bool act_gate = act.flags & gdn::ACT_GATE;
    if (act_gate && (!dA_log || !ddt_bias))
        return fail(GDN_ERR_NULL_ARG, "GDN_ACT_GATE needs the dA_log and ddt_bias outputs");
    if (act_gate && (!aligned4(dA_log) || !aligned4(ddt_bias)))
        return fail(GDN_ERR_MISALIGNED, "dA_log and ddt_bias need 4-byte alignment");
    if (!packed && d->num_seqs != 0)
        return fail(GDN_ERR_BAD_SHAPE, "num_seqs must be 0 without cu_seqlens");
    if (!q || !k || !v || !beta || !g || !dout || !dq || !dk || !dv || !dbeta || !dg || !workspace)
        return fail(GDN_ERR_NULL_ARG,
                    "q, k, v, beta, g, dout, dq, dk, dv, dbeta, dg and workspace are required");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) || !aligned16(dq) ||
        !aligned16(dk) || !aligned16(dv))
        return fail(GDN_ERR_MISALIGNED, "q, k, v, dout, dq, dk, dv need 16-byte alignment");
    if (!aligned4(beta) || !aligned4(g) || !aligned4(h0) || !aligned4(dht) || !aligned4(dbeta) ||
        !aligned4(dg) || !aligned4(dh0) || !aligned8(cu_seqlens))
        return fail(GDN_ERR_MISALIGNED, "float tensors need 4-byte, cu_seqlens 8-byte alignment");
    if (((uintptr_t)workspace & 255u) != 0)
        return fail(GDN_ERR_MISALIGNED, "workspace must be 256-byte aligned");
    BwdLayout L;
    bwd_layout(d, packed, &L);
    if (workspace_bytes < L.total)
        return fail(GDN_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, need %zu", workspace_bytes,
                    L.total);
    hipStream_t st = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    const bool bf16 = d->qkv_dtype == GDN_DTYPE_BF16;
    gdn::ChunkMap map;
    map.max_chunks = L.f.max_chunks;
    map.T = d->seq_len;
    map.nt = (d->seq_len + d->chunk - 1) / d->chunk;
    map.table = packed ? reinterpret_cast<const int4*>(ws + L.f.chunks) : nullptr;
    map.seqs = packed ? reinterpret_cast<const int4*>(ws + L.f.seqs) : nullptr;
    gdn::ChunkWs cw;
    cw.gcum = reinterpret_cast<float*>(ws + L.f.gcum);
    cw.w = ws + L.f.w;
    cw.u = ws + L.f.u;
    cw.qs = ws + L.f.qs;       // Qs^T in the backward mode
    cw.ks = ws + L.f.ks;
    cw.aqk = ws + L.f.aqk;     // Aqk^T in the backward mode
    cw.ainv = reinterpret_cast<float*>(ws + L.f.ainv);
    cw.ksr = ws + L.ksr;
    cw.wt = ws + L.wt;
    const int64_t H = vheads(d), Hq = d->num_heads;   // value heads, q/k heads
    const int64_t N = packed ? d->num_seqs : d->batch;
    const bool gva = H > Hq;
    const bool per_key = d->gate == GDN_GATE_PER_KEY;
    hipError_t e;
    if (packed) {
        gdn::TableLaunch t;
        t.cu_seqlens = cu_seqlens;
        t.N = d->num_seqs;
        t.T = d->seq_len;
        t.C = d->chunk;
        t.table = const_cast<int4*>(map.table);
        t.seqs = const_cast<int4*>(map.seqs);
        t.max_chunks = map.max_chunks;
        t.stream = st;
        if ((e = gdn::launch_table(t)) != hipSuccess) return hip_fail(e, "chunk table launch");
    }
    const bool work = map.max_chunks > 0 && d->seq_len > 0;
    if (work) {   // Step 1: U, W (and the other per-chunk operands) recomputed
        gdn::IntraLaunch a;
        a.q = q;
        a.k = k;
        a.v = v;
        a.beta = beta;
        a.g = g;
        a.map = map;
        a.ws = cw;
        a.H = H;
        a.Hq = Hq;
        a.K = (int)d->key_dim;
        a.V = (int)d->value_dim;
        a.C = d->chunk;
        a.scale = d->scale;
        a.bf16 = bf16;
        a.per_key = per_key;
        a.bwd = true;
        a.act = act;
        a.stream = st;
        if ((e = gdn::launch_intra(a)) != hipSuccess) return hip_fail(e, "intra-chunk launch");
    }
    {   // Step 2: the chunk entry states and V_new recomputed
        gdn::ScanLaunch a;
        a.map = map;
        a.ws = cw;
        a.h0 = h0;
        a.ht = nullptr;
        a.o = nullptr;
        a.hs = ws + L.hs;
        a.vn = ws + L.vn;
        a.N = N;
        a.H = H;
        a.K = (int)d->key_dim;
        a.V = (int)d->value_dim;
        a.C = d->chunk;
        a.bf16 = bf16;
        a.per_key = per_key;
        a.stream = st;
        if ((e = gdn::launch_scan(a)) != hipSuccess) return hip_fail(e, "state pass launch");
    }
    {   // Steps 3-4: the reverse state-gradient recurrence
        gdn::BwdScanLaunch a;
        a.map = map;
        a.gcum = cw.gcum;
        a.ksr = cw.ksr;
        a.aqkt = cw.aqk;
        a.qst = cw.qs;
        a.wt = cw.wt;
        a.dout = dout;
        a.dht = dht;
        a.dh0 = dh0;
        a.dhs = ws + L.dhs;
        a.dvn = ws + L.dvn;
        a.N = N;
        a.H = H;
        a.K = (int)d->key_dim;
        a.V = (int)d->value_dim;
        a.C = d->chunk;
        a.bf16 = bf16;
        a.per_key = per_key;
        a.stream = st;
        if ((e = gdn::launch_bwd_scan(a)) != hipSuccess) return hip_fail(e, "reverse pass launch");
    }
    if (work) {   // Steps 5-6 and the gate
        gdn::BwdLocalLaunch a;
        a.map = map;
        a.q = q;
        a.k = k;
        a.v = v;
        a.dout = dout;
        a.beta = beta;
        a.gcum = cw.gcum;
        a.ainv = cw.ainv;
        a.hs = ws + L.hs;
        a.dhs = ws + L.dhs;
        a.vn = ws + L.vn;
        a.dvn = ws + L.dvn;
        a.dq = dq;
        a.dk = dk;
        a.dv = dv;
        a.dbeta = dbeta;
        a.dg = dg;
        a.dq_part = gva ? reinterpret_cast<float*>(ws + L.dq_part) : nullptr;
        a.dk_part = gva ? reinterpret_cast<float*>(ws + L.dk_part) : nullptr;
        a.act = act;
        a.g = g;
        a.act_part = reinterpret_cast<float*>(ws + L.act_part);
        a.Hq = Hq;
        a.H = H;
        a.K = (int)d->key_dim;
        a.V = (int)d->value_dim;
        a.C = d->chunk;
        a.scale = d->scale;
        a.bf16 = bf16;
        a.per_key = per_key;
        a.stream = st;
        if ((e = gdn::launch_bwd_local(a)) != hipSuccess)
            return hip_fail(e, "per-chunk gradient launch");
        if (gva) {   // dq, dk of each q/k head: the sum over its value heads
            gdn::GvaSumLaunch sl;
            sl.rows = d->batch * d->seq_len;
            sl.H = H;
            sl.Hq = Hq;
            sl.K = (int)d->key_dim;
            sl.bf16 = bf16;
            sl.stream = st;
            sl.part = reinterpret_cast<const float*>(ws + L.dq_part);
            sl.out = dq;
            if ((e = gdn::launch_gva_sum(sl)) != hipSuccess) return hip_fail(e, "dq group sum launch");
            sl.part = reinterpret_cast<const float*>(ws + L.dk_part);
            sl.out = dk;
            if ((e = gdn::launch_gva_sum(sl)) != hipSuccess) return hip_fail(e, "dk group sum launch");
        }
        if (act.flags & gdn::ACT_QK_L2NORM) {   // the normalisation's chain rule, in place
            gdn::L2BwdLaunch l;
            l.rows = d->batch * d->seq_len * Hq;
            l.K = (int)d->key_dim;
            l.bf16 = bf16;
            l.stream = st;
            l.x = q;
            l.dx = dq;
            if ((e = gdn::launch_l2norm_bwd(l)) != hipSuccess) return hip_fail(e, "dq normalisation launch");
            l.x = k;
            l.dx = dk;
            if ((e = gdn::launch_l2norm_bwd(l)) != hipSuccess) return hip_fail(e, "dk normalisation launch");
        }
    }
    if (act_gate) {   // dA_log, ddt_bias (zeros when there are no tokens)
        gdn::ActReduceLaunch r;
        r.map = map;
        if (!work) r.map.max_chunks = 0;
        r.part = reinterpret_cast<const float*>(ws + L.act_part);
        r.dA_log = dA_log;
        r.ddt_bias = ddt_bias;
        r.H = H;
        r.K = per_key ? (int)d->key_dim : 0;
        r.stream = st;
        if ((e = gdn::launch_act_reduce(r)) != hipSuccess) return hip_fail(e, "dA_log sum launch");
    }
    return ok();
}

gdn_status gdn_chunk_bwd(const gdn_fwd_desc* d, const void* q, const void* k, const void* v,
                         const float* beta, const float* g, const float* h0,
                         const int64_t* cu_seqlens, const void* dout, const float* dht,
                         void* dq, void* dk, void* dv, float* dbeta, float* dg, float* dh0,
                         void* workspace, size_t workspace_bytes, void* stream) {
    return gdn_chunk_bwd_act(d, nullptr, q, k, v, beta, g, h0, cu_seqlens, dout, dht, dq, dk, dv,
                             dbeta, dg, dh0, nullptr, nullptr, workspace, workspace_bytes, stream);
}

gdn_status gdn_recurrent_step_act(const gdn_step_desc* d, const gdn_activation* act_in,
                                  const void* q, const void* k, const void* v, const float* beta,
                                  const float* g, float* state, void* o, void* stream) {
    if (!d) return fail(GDN_ERR_NULL_ARG, "desc is NULL");
    gdn::Act act;
    gdn_status s = check_act(act_in, &act);
    if (s != GDN_OK) return s;
    if (d->qkv_dtype != GDN_DTYPE_F32 && d->qkv_dtype != GDN_DTYPE_BF16)
        return fail(GDN_ERR_BAD_DTYPE, "qkv_dtype %d", d->qkv_dtype);
    if (d->gate != GDN_GATE_SCALAR && d->gate != GDN_GATE_PER_KEY)
        return fail(GDN_ERR_BAD_DTYPE, "gate %d", d->gate);
    if (d->num_seqs < 0 || d->num_heads <= 0)
        return fail(GDN_ERR_BAD_SHAPE, "N=%lld H=%lld", (long long)d->num_seqs,
                    (long long)d->num_heads);
    if (!dim_ok(d->key_dim) || !dim_ok(d->value_dim))
        return fail(GDN_ERR_UNSUPPORTED, "K=%lld V=%lld (supported: 64, 128)",
                    (long long)d->key_dim, (long long)d->value_dim);
    if (d->num_v_heads < 0 || (d->num_v_heads > 0 && d->num_v_heads % d->num_heads != 0))
        return fail(GDN_ERR_BAD_SHAPE, "num_v_heads %lld must be 0 or a multiple of num_heads %lld",
                    (long long)d->num_v_heads, (long long)d->num_heads);
    const int64_t HV = d->num_v_heads > 0 ? d->num_v_heads : d->num_heads;
    if (d->num_seqs * HV >= (int64_t)1 << 31)
        return fail(GDN_ERR_BAD_SHAPE, "N*H_V must be below 2^31");
    if (!q || !k || !v || !beta || !g || !state || !o)
        return fail(GDN_ERR_NULL_ARG, "q, k, v, beta, g, state and o are required");
    const size_t es = d->qkv_dtype == GDN_DTYPE_BF16 ? 2 : 4;
    if (!aligned16(state) || ((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) % es ||
        !aligned4(beta) || !aligned4(g))
        return fail(GDN_ERR_MISALIGNED,
                    "state needs 16-byte alignment, the others their element size");
    if (d->num_seqs == 0) return ok();
    gdn::StepLaunch a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.beta = beta;
    a.g = g;
    a.state = state;
    a.o = o;
    a.scale = d->scale;
    a.N = d->num_seqs;
    a.H = HV;
    a.Hq = d->num_heads;
    a.K = (int)d->key_dim;
    a.V = (int)d->value_dim;
    a.bf16 = d->qkv_dtype == GDN_DTYPE_BF16;
    a.per_key = d->gate == GDN_GATE_PER_KEY;
    a.act = act;
    a.stream = static_cast<hipStream_t>(stream);
    hipError_t e = gdn::launch_step(a);
    if (e != hipSuccess) return hip_fail(e, "step launch");
    return ok();
}

gdn_status gdn_recurrent_step(const gdn_step_desc* d, const void* q, const void* k,
                              const void* v, const float* beta, const float* g, float* state,
                              void* o, void* stream) {
    return gdn_recurrent_step_act(d, nullptr, q, k, v, beta, g, state, o, stream);
}

}  // extern "C"
