// Fused chunked forward with the state held in MFMA accumulators, for bf16
// q/k/v with the scalar gate and head sizes K, V in {64, 128}.
//
// One workgroup (8 waves) per (sequence, head, 32-wide value slice) walks the
// chunks of its sequence in order.  Per chunk of n <= C = 64 tokens, with G
// the inclusive cumulative log2-gate inside the chunk and gamma_r = 2^{G_r}
// ("TileLang 实战：KDA 从零到一--Gated DeltaNet" §2.3 eqs. 11-12 and §4.1;
// "Gated Delta Network（GDN）" §4.1(a)-(d)):
//   A_ij   = beta_i 2^{G_i - G_j} k_i.k_j       (j < i)
//   T      = (I + A)^{-1}
//   Aqk_ij = scale 2^{G_i - G_j} q_i.k_j       (j <= i)
//   R      = diag(beta) V - diag(beta gamma) K h
//   V_new  = T R
//   O      = diag(scale gamma) Q h + Aqk V_new
//   h     <- gamma_C h + K^T diag(gamma_C / gamma) V_new
// T R is the pages' U - W h (W = T diag(beta gamma) K, U = T diag(beta) V,
// "TileLang 实战" §2.2.4-2.2.6) taken in the other order, so W and U are never
// formed.  The output reads the state entering the chunk; h is decayed before
// the chunk's contributions are added ("TileLang 实战" §4.4).
//
// The state.  Waves 0 and 1 each own 16 of the 32 value columns and keep
// their K x 16 slice of h in fp32 MFMA accumulators for the whole sequence.
// v_mfma_f32_16x16x32_bf16 contracts over 32 k per instruction, lane group g
// supplying k = 8g..8g+7, and leaves rows 4g..4g+3 of column n of its 16x16
// result in lane 16g+n.  Two result tiles therefore hold, per lane, exactly
// the eight k one lane group supplies to the next instruction, once the k
// are assigned to the tiles' rows in the right order:
//   - over tokens (T R, V_new^T Aqk^T, K^T V_new), the eight k of lane group
//     g of step p are tokens 32p+4g.. and 32p+16+4g.. (rows 4g..4g+3 of token
//     tiles 2p and 2p+1);
//   - over key channels (K h, (Q h)^T), they are channels 32kk+8g..+7, and row
//     4g+e of state tile r is channel 32(r/2) + 8g + 4(r%2) + e.
// So K h, (Q h)^T, T R, V_new^T Aqk^T and K^T V_new take h, R and V_new
// straight from registers: the serial chain from one chunk's state to the
// next touches LDS only for the chunk's own inputs.
//
// The inverse (wave 2): the eight 8x8 diagonal blocks of I + A by forward
// substitution (fp32, one lane per column), one doubling step to the 16x16
// blocks, T_bb = D - D X D (D = the 8x8 inverses, X = the 8x8 block below
// the diagonal), then the off-diagonal 16x16 blocks from
// T_IJ = -T_II sum_{m=J}^{I-1} A_Im T_mJ on bf16 MFMA, every product taken as
// (a matrix in LDS) x (an accumulator) ("阅读笔记：DeltaNet 在 FLA 中的代码实现笔记",
// forward Step 2: small diagonal blocks solved first, combined block-wise;
// "TileLang 实战" §4.2).
//
// Schedule.  Iteration j (one workgroup barrier at its end):
//   waves 0-1   the state pass of chunk j (waits for T_j)
//   wave 2      composes T_j, signals it; inverts the diagonal blocks of
//               chunk j+1 once they are signalled
//   wave 3      the K K^T blocks of chunk j+1 (once its inputs are
//               signalled): the diagonal ones first (signalled), then the
//               off-diagonal ones
//   waves 7,4,5 the causal Q K^T blocks of chunk j+1
//   wave 6      signals that chunk j+1's inputs have landed, derives the
//               gate arrays of chunk j+2 and starts the loads of K, Q, V of
//               chunk j+2 and of g, beta of chunk j+3 straight into LDS
//               (buffer loads with the LDS destination: no registers, rows
//               past a ragged end read as 0)
// Signals are LDS words written with release and polled with acquire
// semantics; every wait is bounded.  The barrier waits for LDS traffic only,
// so the loads stay in flight across it.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

// one instantiation per (K, V); the K = V = 128 one keeps the plain name
namespace fz {
constexpr int K = 128, V = 128;
#include "k_fused_body.hpp"
}  // namespace fz
namespace fz_k128v64 {
constexpr int K = 128, V = 64;
#include "k_fused_body.hpp"
}  // namespace fz_k128v64
namespace fz_k64v128 {
constexpr int K = 64, V = 128;
#include "k_fused_body.hpp"
}  // namespace fz_k64v128
namespace fz_k64v64 {
constexpr int K = 64, V = 64;
#include "k_fused_body.hpp"
}  // namespace fz_k64v64

namespace {
template <int NVT, int NT, auto KF, auto KT>
hipError_t launch_as(const FusedLaunch& a) {
    const int64_t chains = a.N * a.H;
    const int64_t nblk = ((chains + 7) / 8) * 8 * NVT;
    if (a.act.flags & ACT_QK_L2NORM)
        hipLaunchKernelGGL(KT, dim3((unsigned)nblk), dim3(NT), 0, a.stream, a);
    else
        hipLaunchKernelGGL(KF, dim3((unsigned)nblk), dim3(NT), 0, a.stream, a);
    return hipGetLastError();
}
}  // namespace

bool fused_supported(const FusedLaunch& a) {
    return a.bf16 && !a.per_key && (a.K == 64 || a.K == 128) && (a.V == 64 || a.V == 128) && a.C == fz::C;
}

hipError_t launch_fused(const FusedLaunch& a) {
    if (!fused_supported(a)) return hipErrorInvalidValue;
    if (a.K == 128 && a.V == 128)
        return launch_as<fz::NVT, fz::NT, fz::fused_kernel<false>, fz::fused_kernel<true>>(a);
    if (a.K == 128)
        return launch_as<fz_k128v64::NVT, fz_k128v64::NT, fz_k128v64::fused_kernel<false>,
                         fz_k128v64::fused_kernel<true>>(a);
    if (a.V == 128)
        return launch_as<fz_k64v128::NVT, fz_k64v128::NT, fz_k64v128::fused_kernel<false>,
                         fz_k64v128::fused_kernel<true>>(a);
    return launch_as<fz_k64v64::NVT, fz_k64v64::NT, fz_k64v64::fused_kernel<false>,
                     fz_k64v64::fused_kernel<true>>(a);
}

}  // namespace gdn
