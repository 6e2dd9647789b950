// prism_api.hip - C ABI of the PRISM rank-L gated delta-rule forward (see include/prism.h).
//
// Host side only: argument validation, workspace layout, segment sizing and the
// three kernel launches.  Every check runs before anything is enqueued.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "prism.h"
#include "prism_bwd_args.h"
#include "prism_decode.h"
#include "prism_host.h"
#include "prism_kernels.h"
#include "prism_nl.h"

namespace {

using prism::bf16_t;
using prism::FwdArgs;
using prism::host::ChainForm;

constexpr size_t kAlign = 256;
constexpr size_t kCUs = 256;                // compute units of an MI355X
constexpr int kTargetWorkgroupsFast = 256;  // fast sweep: one segment per CU (its LDS fills a CU)

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// a * b with overflow detection (returns false on overflow)
inline bool mul_ok(size_t a, size_t b, size_t* out) {
  if (a != 0 && b > SIZE_MAX / a) return false;
  *out = a * b;
  return true;
}

struct Plan {
  bool fast;     // the bfloat16 d = 64 sweep
  bool fast128;  // the bfloat16 d = 128 half-split sweep
  int P, nch, seg_chunks, nseg;
  size_t off_oloc, off_qhat, off_aagg, off_bagg, off_hin, total;
};

bool valid_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// The specialised sweep (prism_sweep8.h): bfloat16, head dim 64, chunk 64.
// Its loads address one (b, h) pair's slice of u / gamma with 32-bit byte offsets.
bool use_fast(int T, int dk, int dv, int L, int chunk, prism_dtype dt) {
  const size_t slice = (size_t)T * (size_t)(L > 1 ? L - 1 : 1) * 64 * 2;
  return dt == PRISM_BF16 && dk == 64 && dv == 64 && chunk == 64 && slice < ((size_t)1 << 31);
}

// The half-split sweep (prism_sweep128.h): bfloat16, head dim 128, chunk 64, the same
// 32-bit addressing of one pair's u / gamma slice.
bool use_fast128(int T, int dk, int dv, int L, int chunk, prism_dtype dt) {
  const size_t slice = (size_t)T * (size_t)(L > 1 ? L - 1 : 1) * 128 * 2;
  return dt == PRISM_BF16 && dk == 128 && dv == 128 && chunk == 64 && slice < ((size_t)1 << 31);
}

template <class E, int DK, int DV>
constexpr bool fits_c(int C) {
  return C == 16 ? prism::SegLds<E, DK, DV, 16>::fits
         : C == 32 ? prism::SegLds<E, DK, DV, 32>::fits : prism::SegLds<E, DK, DV, 64>::fits;
}

template <class E, int DK>
constexpr bool fits_v(int dv, int C) {
  return dv == 16 ? fits_c<E, DK, 16>(C) : dv == 32 ? fits_c<E, DK, 32>(C)
         : dv == 64 ? fits_c<E, DK, 64>(C) : fits_c<E, DK, 128>(C);
}

template <class E>
constexpr bool fits_e(int dk, int dv, int C) {
  return dk == 16 ? fits_v<E, 16>(dv, C) : dk == 32 ? fits_v<E, 32>(dv, C)
         : dk == 64 ? fits_v<E, 64>(dv, C) : fits_v<E, 128>(dv, C);
}

// Whether the generic sweep's chunk tiles fit the 160 KB of LDS of a CU.
bool lds_fits(prism_dtype dt, int dk, int dv, int C) {
  return dt == PRISM_BF16 ? fits_e<bf16_t>(dk, dv, C) : fits_e<float>(dk, dv, C);
}

// Shape checks shared by the size query and the forward call.
prism_status check_shape(int B, int H, int T, int dk, int dv, int L, int chunk, prism_dtype dt) {
  if (B <= 0 || H <= 0 || T <= 0) return PRISM_ERR_INVALID_ARG;
  if (dt != PRISM_F32 && dt != PRISM_BF16) return PRISM_ERR_INVALID_ARG;
  if (L < 1 || L > 8) return PRISM_ERR_UNSUPPORTED;
  if (!valid_dim(dk) || !valid_dim(dv)) return PRISM_ERR_UNSUPPORTED;
  if (chunk != 16 && chunk != 32 && chunk != 64) return PRISM_ERR_UNSUPPORTED;
  if (!lds_fits(dt, dk, dv, chunk)) return PRISM_ERR_UNSUPPORTED;
  return PRISM_OK;
}

prism_status make_plan(int B, int H, int T, int dk, int dv, int L, int chunk, prism_dtype dt,
                       int seg_chunks, Plan* pl) {
  prism_status st = check_shape(B, H, T, dk, dv, L, chunk, dt);
  if (st != PRISM_OK) return st;
  if (seg_chunks < 0) return PRISM_ERR_INVALID_ARG;
  size_t P;
  if (!mul_ok((size_t)B, (size_t)H, &P) || P > (size_t)INT32_MAX / 2) return PRISM_ERR_INVALID_ARG;
  if (P > 65535) return PRISM_ERR_UNSUPPORTED;  // (b, h) pairs map to grid.y
  const size_t nch = ((size_t)T + chunk - 1) / chunk;
  const bool fast = use_fast(T, dk, dv, L, chunk, dt);
  const bool fast128 = use_fast128(T, dk, dv, L, chunk, dt);
  if (seg_chunks == 0 && fast) {
    size_t nseg_target = kTargetWorkgroupsFast / P;
    if (nseg_target < 1) nseg_target = 1;
    seg_chunks = (int)((nch + nseg_target - 1) / nseg_target);
    if (seg_chunks < 1) seg_chunks = 1;
  } else if (seg_chunks == 0) {
    // the generic and the half-split sweeps run one workgroup per CU (two per segment for
    // the half-split one): the sweep takes about (rounds of kCUs workgroups) x (chunks per
    // segment) chunk times.  The inter-segment scan adds, in chunk times, ~0.1 per segment
    // after a generic sweep; after the half-split one the larger of its chain (~0.19 per
    // segment) and its total work over the GPU (~0.016 per pair and segment), measured at
    // the 130M-layer and 64K-sequence shapes.
    const size_t per_seg = fast128 ? 2 : 1;
    double best = 0.0;
    const size_t smax = nch < 1024 ? nch : 1024;
    for (size_t sc = 1; sc <= smax; ++sc) {
      const size_t ns = (nch + sc - 1) / sc;
      const size_t rounds = (P * ns * per_seg + kCUs - 1) / kCUs;
      const double scan = fast128 ? std::max(0.19 * (double)ns, 0.016 * (double)(P * ns)) : 0.1 * (double)ns;
      const double cost = (double)rounds * (double)sc + scan;
      if (sc == 1 || cost < best) {
        best = cost;
        seg_chunks = (int)sc;
      }
    }
  }
  const size_t nseg = (nch + seg_chunks - 1) / seg_chunks;
  // O_loc and Qhat in the I/O type (the d = 64 fast path's in fragment order); H_in in
  // bfloat16 on the fast paths (the corrections' MFMA operand), float32 on the generic path
  const size_t wel = dt == PRISM_BF16 ? 2 : 4, hel = fast || fast128 ? 2 : 4;
  size_t Tpad = nch * (size_t)chunk, a, b, c;
  size_t sz_oloc, sz_qhat, sz_agg_a, sz_agg_b, sz_hin;
  if (!mul_ok(P, Tpad, &a) || !mul_ok(a, (size_t)dv * wel, &sz_oloc)) return PRISM_ERR_INVALID_ARG;
  if (!mul_ok(a, (size_t)dk * wel, &sz_qhat)) return PRISM_ERR_INVALID_ARG;
  if (!mul_ok(P, nseg, &b) || !mul_ok(b, (size_t)dk * dk * 4, &sz_agg_a)) return PRISM_ERR_INVALID_ARG;
  if (!mul_ok(b, (size_t)dk * dv * 4, &sz_agg_b)) return PRISM_ERR_INVALID_ARG;
  sz_hin = sz_agg_b / 4 * hel;
  // inputs must be addressable too: P*T*(L-1)*max(dk,dv) elements
  if (!mul_ok(P, (size_t)T, &c) || !mul_ok(c, (size_t)L * (dk > dv ? dk : dv) * 4, &c))
    return PRISM_ERR_INVALID_ARG;
  pl->fast = fast;
  pl->fast128 = fast128;
  pl->P = (int)P;
  pl->nch = (int)nch;
  pl->seg_chunks = seg_chunks;
  pl->nseg = (int)nseg;
  pl->off_oloc = 0;
  pl->off_qhat = align_up(pl->off_oloc + sz_oloc);
  pl->off_aagg = align_up(pl->off_qhat + sz_qhat);
  pl->off_bagg = align_up(pl->off_aagg + sz_agg_a);
  pl->off_hin = align_up(pl->off_bagg + sz_agg_b);
  pl->total = align_up(pl->off_hin + sz_hin);
  if (pl->total < sz_oloc) return PRISM_ERR_INVALID_ARG;
  return PRISM_OK;
}

// The generic forward of one I/O type, by key width.
prism_status dispatch_generic(prism_dtype dt, int dk, int dv, int C, const FwdArgs& a,
                              const prism::host::LaunchShape& s, hipEvent_t* ev, hipStream_t st) {
  using namespace prism::host;
  if (dt == PRISM_BF16) {
    switch (dk) {
      case 16: return launch_generic_bf16_dk16(dv, C, a, s, ev, st);
      case 32: return launch_generic_bf16_dk32(dv, C, a, s, ev, st);
      case 64: return launch_generic_bf16_dk64(dv, C, a, s, ev, st);
      default: return launch_generic_bf16_dk128(dv, C, a, s, ev, st);
    }
  }
  switch (dk) {
    case 16: return launch_generic_f32_dk16(dv, C, a, s, ev, st);
    case 32: return launch_generic_f32_dk32(dv, C, a, s, ev, st);
    case 64: return launch_generic_f32_dk64(dv, C, a, s, ev, st);
    default: return launch_generic_f32_dk128(dv, C, a, s, ev, st);
  }
}

prism_status fwd_impl(const void* q, const void* k, const void* v, const float* g, const float* beta,
                      const void* u, const float* alpha, const void* gamma, const float* conv_w,
                      int B, int H, int T, int dk, int dv, int L, int chunk, prism_dtype dt,
                      void* o, float* S_final, void* workspace, size_t workspace_bytes,
                      int seg_chunks, hipEvent_t* ev, hipStream_t stream,
                      const float* S0 = nullptr, const void* conv_in = nullptr, void* conv_out = nullptr,
                      ChainForm form = ChainForm::kLinear) {
  Plan pl;
  prism_status st = make_plan(B, H, T, dk, dv, L, chunk, dt, seg_chunks, &pl);
  if (st != PRISM_OK) return st;
  if (!q || !k || !v || !g || !beta || !o || !S_final) return PRISM_ERR_INVALID_ARG;
  if (L > 1 && (!u || !alpha || !gamma || !conv_w)) return PRISM_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < pl.total) return PRISM_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.u = u; a.gamma = gamma;
  a.g = g; a.beta = beta; a.alpha = alpha; a.conv_w = conv_w;
  a.o = o; a.S_final = S_final;
  a.S0 = S0; a.conv_in = conv_in; a.conv_out = conv_out;
  a.Oloc = reinterpret_cast<float*>(ws + pl.off_oloc);
  a.Qhat = reinterpret_cast<float*>(ws + pl.off_qhat);
  a.Aagg = reinterpret_cast<float*>(ws + pl.off_aagg);
  a.Bagg = reinterpret_cast<float*>(ws + pl.off_bagg);
  a.Hin = reinterpret_cast<float*>(ws + pl.off_hin);
  a.B = B; a.H = H; a.T = T; a.L = L;
  a.nch = pl.nch; a.seg_chunks = pl.seg_chunks; a.nseg = pl.nseg;
  a.chain_delta = form == ChainForm::kDelta ? 1 : 0;
  if (form == ChainForm::kGelu && !pl.fast && !pl.fast128) return PRISM_ERR_UNSUPPORTED;
  const prism::host::LaunchShape shape{pl.P, pl.nch, pl.nseg};
  if (pl.fast)
    st = prism::host::launch_fast(a, shape, ev, stream, L > 1 ? form : ChainForm::kLinear);
  else if (pl.fast128)
    st = prism::host::launch_fast128(a, shape, ev, stream, L > 1 ? form : ChainForm::kLinear);
  else
    st = dispatch_generic(dt, dk, dv, chunk, a, shape, ev, stream);
  if (st != PRISM_OK || conv_out == nullptr) return st;
  // after the sweep, the only reader of conv_in, so conv_out may alias it
  if (dt == PRISM_BF16)
    hipLaunchKernelGGL((prism::conv_tail_kernel<bf16_t>), dim3(pl.P), dim3(128), 0, stream, a, dv);
  else
    hipLaunchKernelGGL((prism::conv_tail_kernel<float>), dim3(pl.P), dim3(128), 0, stream, a, dv);
  return hipGetLastError() == hipSuccess ? PRISM_OK : PRISM_ERR_HIP;
}

template <class E>
prism_status decode_dispatch(int d, const prism::DecodeArgs& a, int P, hipStream_t stream) {
  switch (d) {
    case 16: hipLaunchKernelGGL((prism::decode_kernel<E, 16>), dim3(P), dim3(256), 0, stream, a); break;
    case 32: hipLaunchKernelGGL((prism::decode_kernel<E, 32>), dim3(P), dim3(256), 0, stream, a); break;
    case 64: hipLaunchKernelGGL((prism::decode_kernel<E, 64>), dim3(P), dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL((prism::decode_kernel<E, 128>), dim3(P), dim3(256), 0, stream, a); break;
  }
  return hipGetLastError() == hipSuccess ? PRISM_OK : PRISM_ERR_HIP;
}

// Workspace of the backward, float32 regions aligned to 256 bytes.
//   sequential: checkpoints [P][NSP][nblk][D*D/NSP], block states [P][NSP][64][D*D/NSP],
//     dconv_w shares [P][4][D] and, with NSP = D/16 > 1 workgroups per pair, their per-token
//     column sums [P][NSP][T][RED];
//   segment-parallel: B, Phi, ell, S_in, Lambda [P][nseg][D][D] each, sub-block checkpoints
//     [P][nseg][seg_len/8][D][D], sub-block states [P][nseg][8][D][D], dconv_w shares
//     [P][nseg][4][D], anchor carries [P][nseg][3][D] and, with NSP > 1 workgroups per
//     state, the column sums [P][NSP][T][RED].
struct BwdPlan {
  int P, nblk, nseg, seg_len;
  bool segments;
  size_t off_ckpt, off_scr, off_part, off_red, off_seg, off_carry, total;
};

// rank slots compiled in for L (0 for L = 1, 3 for L <= 4, 7 for L <= 8)
inline int bwd_rank_slots(int L) { return L == 1 ? 0 : L <= 4 ? 3 : 7; }

// Segment length of the segment-parallel backward when the caller does not give one: the
// longest of 128, 64, 32 tokens that still makes at least 2048 workgroups (several per
// CU, so that their token steps hide one another's latency), else 16.
int bwd_default_seg_len(size_t P, int T, int d) {
  const size_t nsp = (size_t)prism::host::bwd_seg_slices(d);
  for (int len = 128; len >= 32; len /= 2)
    if (P * (((size_t)T + len - 1) / len) * nsp >= 2048) return len;
  return 16;
}

// seg_len: 0 for the sequential form, else the segment length (a multiple of 8, >= 16).
prism_status make_bwd_plan(int B, int H, int T, int dk, int dv, int L, prism_dtype dt, int seg_len, BwdPlan* pl) {
  if (B <= 0 || H <= 0 || T <= 0) return PRISM_ERR_INVALID_ARG;
  if (dt != PRISM_F32 && dt != PRISM_BF16) return PRISM_ERR_INVALID_ARG;
  if (L < 1 || L > 8) return PRISM_ERR_UNSUPPORTED;
  if (!valid_dim(dk) || dk != dv) return PRISM_ERR_UNSUPPORTED;
  if (seg_len != 0 && (seg_len < 16 || seg_len % prism::kBwdSegSub != 0)) return PRISM_ERR_INVALID_ARG;
  size_t P, a, c, sz_ckpt, sz_scr, sz_part, sz_seg = 0, sz_carry = 0;
  if (!mul_ok((size_t)B, (size_t)H, &P) || P > (size_t)INT32_MAX) return PRISM_ERR_INVALID_ARG;
  // inputs must be addressable: P*T*L*dk elements
  if (!mul_ok(P, (size_t)T, &c) || !mul_ok(c, (size_t)L * dk * 4, &c)) return PRISM_ERR_INVALID_ARG;
  const size_t dd = (size_t)dk * dk * 4;
  const bool seg = seg_len != 0;
  const size_t nseg = seg ? ((size_t)T + seg_len - 1) / seg_len : 1;
  const size_t nblk = ((size_t)T + prism::kBwdBlock - 1) / prism::kBwdBlock;
  int nsp = dk / 16;
  if (seg) {
    nsp = prism::host::bwd_seg_slices(dk);
    size_t ps;
    if (!mul_ok(P, nseg, &ps) || ps * nsp > (size_t)INT32_MAX) return PRISM_ERR_INVALID_ARG;
    if (!mul_ok(ps, dd, &a) || !mul_ok(a, 5, &sz_seg)) return PRISM_ERR_INVALID_ARG;
    if (!mul_ok(a, (size_t)seg_len / prism::kBwdSegSub, &sz_ckpt)) return PRISM_ERR_INVALID_ARG;
    if (!mul_ok(a, (size_t)prism::kBwdSegSub, &sz_scr)) return PRISM_ERR_INVALID_ARG;
    if (!mul_ok(ps, (size_t)4 * dk * 4, &sz_part) || !mul_ok(ps, (size_t)3 * dk * 4, &sz_carry))
      return PRISM_ERR_INVALID_ARG;
  } else {
    if (!mul_ok(P, nblk, &a) || !mul_ok(a, dd, &sz_ckpt)) return PRISM_ERR_INVALID_ARG;
    if (!mul_ok(P, (size_t)prism::kBwdBlock, &a) || !mul_ok(a, dd, &sz_scr)) return PRISM_ERR_INVALID_ARG;
    if (!mul_ok(P, (size_t)4 * dk * 4, &sz_part)) return PRISM_ERR_INVALID_ARG;
  }
  // per-workgroup column sums when a state's rows span more than one workgroup
  size_t sz_red = 0;
  const int nr = bwd_rank_slots(L) > 0 ? bwd_rank_slots(L) : 1;
  if (nsp > 1) {
    const size_t red = (size_t)(2 + nr) * dk + 3 + nr;
    size_t x;
    if (!mul_ok(P, (size_t)nsp * T, &x) || !mul_ok(x, red * 4, &sz_red)) return PRISM_ERR_INVALID_ARG;
  }
  pl->P = (int)P;
  pl->nblk = (int)nblk;
  pl->nseg = (int)nseg;
  pl->seg_len = seg_len;
  pl->segments = seg;
  pl->off_ckpt = 0;
  pl->off_scr = align_up(sz_ckpt);
  pl->off_part = align_up(pl->off_scr + sz_scr);
  pl->off_red = align_up(pl->off_part + sz_part);
  pl->off_seg = align_up(pl->off_red + sz_red);
  pl->off_carry = align_up(pl->off_seg + sz_seg);
  pl->total = align_up(pl->off_carry + sz_carry);
  if (pl->total < sz_ckpt + sz_scr + sz_red + sz_seg) return PRISM_ERR_INVALID_ARG;
  return PRISM_OK;
}

// the default segment length for the shape (0 when the shape is refused)
int bwd_seg_len_for(int B, int H, int T, int dk) {
  if (B <= 0 || H <= 0 || T <= 0 || !valid_dim(dk)) return 0;
  return bwd_default_seg_len((size_t)B * (size_t)H, T, dk);
}

}  // namespace

extern "C" {

size_t prism_bwd_workspace_bytes(int B, int H, int T, int dk, int dv, int L, prism_dtype dt) {
  BwdPlan pl;
  const int len = bwd_seg_len_for(B, H, T, dk);
  return len > 0 && make_bwd_plan(B, H, T, dk, dv, L, dt, len, &pl) == PRISM_OK ? pl.total : 0;
}

size_t prism_bwd_seg_workspace_bytes(int B, int H, int T, int dk, int dv, int L, prism_dtype dt, int seg_len) {
  BwdPlan pl;
  return seg_len > 0 && make_bwd_plan(B, H, T, dk, dv, L, dt, seg_len, &pl) == PRISM_OK ? pl.total : 0;
}

size_t prism_bwd_lowmem_workspace_bytes(int B, int H, int T, int dk, int dv, int L, prism_dtype dt) {
  BwdPlan pl;
  return make_bwd_plan(B, H, T, dk, dv, L, dt, 0, &pl) == PRISM_OK ? pl.total : 0;
}

}  // extern "C"

namespace {

prism_status bwd_impl(const void* q, const void* k, const void* v, const float* g, const float* beta,
                      const void* u, const float* alpha, const void* gamma, const float* conv_w,
                      int B, int H, int T, int dk, int dv, int L, prism_dtype dt,
                      const void* d_o, const float* dS_final,
                      float* dq, float* dk_out, float* dv_out, float* dg, float* dbeta,
                      float* du, float* dalpha, float* dgamma, float* dconv_w,
                      void* workspace, size_t workspace_bytes, hipStream_t stream, int seg_len) {
  BwdPlan pl;
  prism_status st = make_bwd_plan(B, H, T, dk, dv, L, dt, seg_len, &pl);
  if (st != PRISM_OK) return st;
  if (!q || !k || !v || !g || !beta || !d_o || !dq || !dk_out || !dv_out || !dg || !dbeta)
    return PRISM_ERR_INVALID_ARG;
  if (L > 1 && (!u || !alpha || !gamma || !conv_w || !du || !dalpha || !dgamma || !dconv_w))
    return PRISM_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < pl.total) return PRISM_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  prism::BwdArgs a = {};
  a.q = q; a.k = k; a.v = v; a.u = u; a.gamma = gamma; a.d_o = d_o;
  a.g = g; a.beta = beta; a.alpha = alpha; a.conv_w = conv_w; a.dS_final = dS_final;
  a.dq = dq; a.dk = dk_out; a.dv = dv_out; a.dg = dg; a.dbeta = dbeta;
  a.du = du; a.dalpha = dalpha; a.dgamma = dgamma;
  a.ckpt = reinterpret_cast<float*>(ws + pl.off_ckpt);
  a.scratch = reinterpret_cast<float*>(ws + pl.off_scr);
  a.dconv_part = reinterpret_cast<float*>(ws + pl.off_part);
  a.part = reinterpret_cast<float*>(ws + pl.off_red);
  const size_t sq = (size_t)pl.P * pl.nseg * dk * dk;
  float* sg = reinterpret_cast<float*>(ws + pl.off_seg);
  a.seg_B = pl.segments ? sg : nullptr;
  a.seg_Phi = pl.segments ? sg + sq : nullptr;
  a.seg_ell = pl.segments ? sg + 2 * sq : nullptr;
  a.seg_Sin = pl.segments ? sg + 3 * sq : nullptr;
  a.seg_Lam = pl.segments ? sg + 4 * sq : nullptr;
  a.carry = pl.segments ? reinterpret_cast<float*>(ws + pl.off_carry) : nullptr;
  a.H = H; a.T = T; a.L = L; a.nblk = pl.nblk;
  a.nseg = pl.nseg; a.seg_len = pl.seg_len;
  return prism::host::launch_bwd(dt, dk, a, B, pl.P, dconv_w, pl.segments, stream);
}

}  // namespace

extern "C" {

prism_status prism_bwd(const void* q, const void* k, const void* v, const float* g, const float* beta,
                       const void* u, const float* alpha, const void* gamma, const float* conv_w,
                       int B, int H, int T, int dk, int dv, int L, prism_dtype dt,
                       const void* d_o, const float* dS_final,
                       float* dq, float* dk_out, float* dv_out, float* dg, float* dbeta,
                       float* du, float* dalpha, float* dgamma, float* dconv_w,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const int len = bwd_seg_len_for(B, H, T, dk);
  if (len == 0) return B <= 0 || H <= 0 || T <= 0 ? PRISM_ERR_INVALID_ARG : PRISM_ERR_UNSUPPORTED;
  return bwd_impl(q, k, v, g, beta, u, alpha, gamma, conv_w, B, H, T, dk, dv, L, dt, d_o, dS_final, dq, dk_out,
                  dv_out, dg, dbeta, du, dalpha, dgamma, dconv_w, workspace, workspace_bytes, stream, len);
}

prism_status prism_bwd_seg(const void* q, const void* k, const void* v, const float* g, const float* beta,
                           const void* u, const float* alpha, const void* gamma, const float* conv_w,
                           int B, int H, int T, int dk, int dv, int L, prism_dtype dt,
                           const void* d_o, const float* dS_final,
                           float* dq, float* dk_out, float* dv_out, float* dg, float* dbeta,
                           float* du, float* dalpha, float* dgamma, float* dconv_w, int seg_len,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (seg_len <= 0) return PRISM_ERR_INVALID_ARG;
  return bwd_impl(q, k, v, g, beta, u, alpha, gamma, conv_w, B, H, T, dk, dv, L, dt, d_o, dS_final, dq, dk_out,
                  dv_out, dg, dbeta, du, dalpha, dgamma, dconv_w, workspace, workspace_bytes, stream, seg_len);
}

prism_status prism_bwd_lowmem(const void* q, const void* k, const void* v, const float* g, const float* beta,
                              const void* u, const float* alpha, const void* gamma, const float* conv_w,
                              int B, int H, int T, int dk, int dv, int L, prism_dtype dt,
                              const void* d_o, const float* dS_final,
                              float* dq, float* dk_out, float* dv_out, float* dg, float* dbeta,
                              float* du, float* dalpha, float* dgamma, float* dconv_w,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return bwd_impl(q, k, v, g, beta, u, alpha, gamma, conv_w, B, H, T, dk, dv, L, dt, d_o, dS_final, dq, dk_out,
                  dv_out, dg, dbeta, du, dalpha, dgamma, dconv_w, workspace, workspace_bytes, stream, 0);
}

}  // extern "C"

namespace {

// Workspace of the chunked backward: per 64-token chunk two float32 64 x 64 matrices (end
// state from zero, local adjoint) and three bf16 ones (operator, entering state, arriving
// adjoint), its anchor carry [3][64] and dconv_w share [4][64], and 3 + L bf16 64 x 64
// matrices (T, Uc, Wc, V' and the chain residuals r_0 .. r_{L-2}) that the local pass hands
// to the gradient pass; per group of four chunks six float32 64 x 64 matrices for the
// two-level scan.
struct BwdChunkPlan {
  int P, nch, ngrp;
  size_t off_seg, off_carry, off_part, off_mats, off_grp, total;
};

prism_status make_bwd_chunk_plan(int B, int H, int T, int dk, int dv, int L, prism_dtype dt, BwdChunkPlan* pl) {
  if (B <= 0 || H <= 0 || T <= 0) return PRISM_ERR_INVALID_ARG;
  if (dt != PRISM_F32 && dt != PRISM_BF16) return PRISM_ERR_INVALID_ARG;
  if (L < 1 || L > 8) return PRISM_ERR_UNSUPPORTED;
  if (dt != PRISM_BF16 || dk != 64 || dv != 64) return PRISM_ERR_UNSUPPORTED;
  size_t P, c, nseg_all, sz_seg, sz_carry, sz_part, sz_mats, sz_grp;
  if (!mul_ok((size_t)B, (size_t)H, &P) || P > 65535) return PRISM_ERR_INVALID_ARG;
  if (!mul_ok(P, (size_t)T, &c) || !mul_ok(c, (size_t)L * dk * 4, &c)) return PRISM_ERR_INVALID_ARG;
  const size_t nch = ((size_t)T + 63) / 64;
  if (!mul_ok(P, nch, &nseg_all) || nseg_all > (size_t)INT32_MAX) return PRISM_ERR_INVALID_ARG;
  if (!mul_ok(nseg_all, (size_t)(2 * 4 + 3 * 2) * 64 * 64, &sz_seg) || !mul_ok(nseg_all, (size_t)3 * 64 * 4, &sz_carry) ||
      !mul_ok(nseg_all, (size_t)4 * 64 * 4, &sz_part) || !mul_ok(nseg_all, (size_t)(3 + L) * 64 * 64 * 2, &sz_mats))
    return PRISM_ERR_INVALID_ARG;
  const size_t ngrp = (nch + prism::kBwdGroup - 1) / prism::kBwdGroup;
  if (!mul_ok(P * ngrp, (size_t)6 * 64 * 64 * 4, &sz_grp)) return PRISM_ERR_INVALID_ARG;
  pl->P = (int)P;
  pl->nch = (int)nch;
  pl->off_seg = 0;
  pl->off_carry = align_up(sz_seg);
  pl->off_part = align_up(pl->off_carry + sz_carry);
  pl->off_mats = align_up(pl->off_part + sz_part);
  pl->off_grp = align_up(pl->off_mats + sz_mats);
  pl->total = align_up(pl->off_grp + sz_grp);
  pl->ngrp = (int)ngrp;
  return PRISM_OK;
}

}  // namespace

extern "C" {

size_t prism_bwd_chunked_workspace_bytes(int B, int H, int T, int dk, int dv, int L, prism_dtype dt) {
  BwdChunkPlan pl;
  return make_bwd_chunk_plan(B, H, T, dk, dv, L, dt, &pl) == PRISM_OK ? pl.total : 0;
}

prism_status prism_bwd_chunked(const void* q, const void* k, const void* v, const float* g, const float* beta,
                               const void* u, const float* alpha, const void* gamma, const float* conv_w,
                               int B, int H, int T, int dk, int dv, int L, prism_dtype dt,
                               const void* d_o, const float* dS_final,
                               float* dq, float* dk_out, float* dv_out, float* dg, float* dbeta,
                               float* du, float* dalpha, float* dgamma, float* dconv_w,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  BwdChunkPlan pl;
  prism_status st = make_bwd_chunk_plan(B, H, T, dk, dv, L, dt, &pl);
  if (st != PRISM_OK) return st;
  if (!q || !k || !v || !g || !beta || !d_o || !dq || !dk_out || !dv_out || !dg || !dbeta)
    return PRISM_ERR_INVALID_ARG;
  if (L > 1 && (!u || !alpha || !gamma || !conv_w || !du || !dalpha || !dgamma || !dconv_w))
    return PRISM_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < pl.total) return PRISM_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  prism::BwdArgs a = {};
  a.q = q; a.k = k; a.v = v; a.u = u; a.gamma = gamma; a.d_o = d_o;
  a.g = g; a.beta = beta; a.alpha = alpha; a.conv_w = conv_w; a.dS_final = dS_final;
  a.dq = dq; a.dk = dk_out; a.dv = dv_out; a.dg = dg; a.dbeta = dbeta;
  a.du = du; a.dalpha = dalpha; a.dgamma = dgamma;
  const size_t sq = (size_t)pl.P * pl.nch * 64 * 64;
  float* sg = reinterpret_cast<float*>(ws + pl.off_seg);
  a.seg_B = sg;
  a.seg_ell = sg + sq;
  bf16_t* sb = reinterpret_cast<bf16_t*>(sg + 2 * sq);
  a.c_Acc = sb;
  a.c_Sin = sb + sq;
  a.c_Lam = sb + 2 * sq;
  a.carry = reinterpret_cast<float*>(ws + pl.off_carry);
  a.dconv_part = reinterpret_cast<float*>(ws + pl.off_part);
  a.chunk_mats = ws + pl.off_mats;
  const size_t gq = (size_t)pl.P * pl.ngrp * 64 * 64;
  float* gs = reinterpret_cast<float*>(ws + pl.off_grp);
  a.grp_Acc = gs;
  a.grp_Phi = gs + gq;
  a.grp_B = gs + 2 * gq;
  a.grp_ell = gs + 3 * gq;
  a.grp_Sin = gs + 4 * gq;
  a.grp_Lam = gs + 5 * gq;
  a.ngrp = pl.ngrp;
  a.H = H; a.T = T; a.L = L; a.nblk = 0;
  a.nseg = pl.nch; a.seg_len = 64;
  return prism::host::launch_bwd_chunked(a, B, pl.P, dconv_w, stream);
}


size_t prism_fwd_workspace_bytes(int B, int H, int T, int dk, int dv, int L, int chunk, prism_dtype dt) {
  Plan pl;
  return make_plan(B, H, T, dk, dv, L, chunk, dt, 0, &pl) == PRISM_OK ? pl.total : 0;
}

size_t prism_fwd_seg_workspace_bytes(int B, int H, int T, int dk, int dv, int L, int chunk, prism_dtype dt,
                                     int seg_chunks) {
  Plan pl;
  return make_plan(B, H, T, dk, dv, L, chunk, dt, seg_chunks, &pl) == PRISM_OK ? pl.total : 0;
}

prism_status prism_fwd(const void* q, const void* k, const void* v, const float* g, const float* beta,
                       const void* u, const float* alpha, const void* gamma, const float* conv_w,
                       int B, int H, int T, int dk, int dv, int L, int chunk, prism_dtype dt,
                       void* o, float* S_final, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return fwd_impl(q, k, v, g, beta, u, alpha, gamma, conv_w, B, H, T, dk, dv, L, chunk, dt, o, S_final,
                  workspace, workspace_bytes, 0, nullptr, stream);
}

prism_status prism_fwd_timed(const void* q, const void* k, const void* v, const float* g, const float* beta,
                             const void* u, const float* alpha, const void* gamma, const float* conv_w,
                             int B, int H, int T, int dk, int dv, int L, int chunk, prism_dtype dt,
                             void* o, float* S_final, void* workspace, size_t workspace_bytes,
                             hipEvent_t* events, hipStream_t stream) {
  if (!events) return PRISM_ERR_INVALID_ARG;
  return fwd_impl(q, k, v, g, beta, u, alpha, gamma, conv_w, B, H, T, dk, dv, L, chunk, dt, o, S_final,
                  workspace, workspace_bytes, 0, events, stream);
}

prism_status prism_fwd_state(const void* q, const void* k, const void* v, const float* g, const float* beta,
                             const void* u, const float* alpha, const void* gamma, const float* conv_w,
                             int B, int H, int T, int dk, int dv, int L, int chunk, prism_dtype dt,
                             const float* S0, const void* conv_in,
                             void* o, float* S_final, void* conv_out,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return fwd_impl(q, k, v, g, beta, u, alpha, gamma, conv_w, B, H, T, dk, dv, L, chunk, dt, o, S_final,
                  workspace, workspace_bytes, 0, nullptr, stream, S0, conv_in, conv_out);
}

prism_status prism_decode_step(const void* q, const void* k, const void* v, const float* g, const float* beta,
                               const void* u, const float* alpha, const void* gamma, const float* conv_w,
                               int B, int H, int dk, int dv, int L, prism_dtype dt,
                               float* S, void* conv_state, void* o, hipStream_t stream) {
  if (B <= 0 || H <= 0) return PRISM_ERR_INVALID_ARG;
  if (!(dk == dv && (dk == 16 || dk == 32 || dk == 64 || dk == 128))) return PRISM_ERR_UNSUPPORTED;
  if (L < 1 || L > 8 || (dt != PRISM_F32 && dt != PRISM_BF16)) return PRISM_ERR_UNSUPPORTED;
  if (!q || !k || !v || !g || !beta || !S || !o) return PRISM_ERR_INVALID_ARG;
  if (L > 1 && (!u || !alpha || !gamma || !conv_w || !conv_state)) return PRISM_ERR_INVALID_ARG;
  size_t P;
  if (!mul_ok((size_t)B, (size_t)H, &P) || P > 0x7fffffff) return PRISM_ERR_INVALID_ARG;
  prism::DecodeArgs a;
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
  a.u = u; a.alpha = alpha; a.gamma = gamma; a.conv_w = conv_w;
  a.S = S; a.conv_state = conv_state; a.o = o;
  a.H = H; a.L = L;
  return dt == PRISM_BF16 ? decode_dispatch<bf16_t>(dk, a, (int)P, stream)
                          : decode_dispatch<float>(dk, a, (int)P, stream);
}

prism_status prism_fwd_seg(const void* q, const void* k, const void* v, const float* g, const float* beta,
                           const void* u, const float* alpha, const void* gamma, const float* conv_w,
                           int B, int H, int T, int dk, int dv, int L, int chunk, prism_dtype dt,
                           void* o, float* S_final, void* workspace, size_t workspace_bytes,
                           int seg_chunks, hipStream_t stream) {
  if (seg_chunks <= 0) return PRISM_ERR_INVALID_ARG;
  return fwd_impl(q, k, v, g, beta, u, alpha, gamma, conv_w, B, H, T, dk, dv, L, chunk, dt, o, S_final,
                  workspace, workspace_bytes, seg_chunks, nullptr, stream);
}

// Bytes of the chain factors of the nonlinear refinement: B H T (L-1) dv elements of dt.
static bool nl_gamma_bytes(int B, int H, int T, int dv, int L, prism_dtype dt, size_t* out) {
  size_t P, pt;
  if (!mul_ok((size_t)B, (size_t)H, &P) || !mul_ok(P, (size_t)T, &pt)) return false;
  return mul_ok(pt, (size_t)(L - 1) * dv * (dt == PRISM_BF16 ? 2 : 4), out);
}

}  // extern "C"

namespace {

// The chain-factor pass: linear chain (alpha read) or written corrections (delta).
prism_status gain_impl(const void* v, const float* alpha, const void* p, const float* conv_w,
                       const void* conv_in, int B, int H, int T, int dv, int L, prism_dtype dt,
                       void* gamma, bool delta, hipStream_t stream) {
  if (B <= 0 || H <= 0 || T <= 0) return PRISM_ERR_INVALID_ARG;
  if (dt != PRISM_F32 && dt != PRISM_BF16) return PRISM_ERR_INVALID_ARG;
  if (L < 1 || L > 8 || !valid_dim(dv)) return PRISM_ERR_UNSUPPORTED;
  if (L == 1) return PRISM_OK;
  if (!v || (!delta && !alpha) || !p || !conv_w || !gamma) return PRISM_ERR_INVALID_ARG;
  size_t P, bytes;
  if (!mul_ok((size_t)B, (size_t)H, &P) || !nl_gamma_bytes(B, H, T, dv, L, dt, &bytes)) return PRISM_ERR_INVALID_ARG;
  if (P > 65535) return PRISM_ERR_UNSUPPORTED;  // (b, h) pairs map to grid.y, as in the forward
  const int lognc = dv == 16 ? 2 : dv == 32 ? 3 : dv == 64 ? 4 : 5;
  const size_t groups = (size_t)T << lognc;    // < 2^36: T < 2^31, dv / 4 <= 32
  if (groups > (size_t)UINT32_MAX - 255) return PRISM_ERR_UNSUPPORTED;
  const dim3 grid((unsigned)((groups + 255) / 256), (unsigned)P);
  prism::NlArgs a;
  a.v = v; a.alpha = alpha; a.p = p; a.conv_w = conv_w; a.conv_in = conv_in; a.gamma = gamma;
  a.H = H; a.T = T; a.L = L; a.dv = dv; a.lognc = lognc;
  return prism::host::launch_gain(a, dt, grid, delta, stream);
}

}  // namespace

extern "C" {

prism_status prism_nl_gain(const void* v, const float* alpha, const void* p, const float* conv_w,
                           const void* conv_in, int B, int H, int T, int dv, int L, prism_dtype dt,
                           void* gamma, hipStream_t stream) {
  return gain_impl(v, alpha, p, conv_w, conv_in, B, H, T, dv, L, dt, gamma, false, stream);
}

prism_status prism_delta_gain(const void* v, const void* p, const float* conv_w, const void* conv_in,
                              int B, int H, int T, int dv, int L, prism_dtype dt, void* gamma,
                              hipStream_t stream) {
  return gain_impl(v, nullptr, p, conv_w, conv_in, B, H, T, dv, L, dt, gamma, true, stream);
}

size_t prism_fwd_nl_workspace_bytes(int B, int H, int T, int dk, int dv, int L, int chunk, prism_dtype dt) {
  Plan pl;
  size_t gb;
  if (make_plan(B, H, T, dk, dv, L, chunk, dt, 0, &pl) != PRISM_OK || !nl_gamma_bytes(B, H, T, dv, L, dt, &gb))
    return 0;
  return align_up(gb) + pl.total;
}

}  // extern "C"

namespace {

// prism_fwd_nl with a segment length in chunks (0 = the planner's choice).
prism_status fwd_nl_impl(const void* q, const void* k, const void* v, const float* g, const float* beta,
                         const void* u, const float* alpha, const void* p, const float* conv_w,
                         int B, int H, int T, int dk, int dv, int L, int chunk, prism_dtype dt,
                         void* o, float* S_final, void* workspace, size_t workspace_bytes, int seg_chunks,
                         hipStream_t stream) {
  // every check before the first launch
  Plan pl;
  prism_status st = make_plan(B, H, T, dk, dv, L, chunk, dt, seg_chunks, &pl);
  if (st != PRISM_OK) return st;
  if (!q || !k || !v || !g || !beta || !o || !S_final) return PRISM_ERR_INVALID_ARG;
  if (L > 1 && (!u || !alpha || !p || !conv_w)) return PRISM_ERR_INVALID_ARG;
  size_t gb;
  if (!nl_gamma_bytes(B, H, T, dv, L, dt, &gb)) return PRISM_ERR_INVALID_ARG;
  const size_t off = align_up(gb);
  if (!workspace || workspace_bytes < off + pl.total) return PRISM_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  // the bf16 d = 64 and d = 128 sweeps evaluate the factors in their own residual chain:
  // no factor pass
  if ((pl.fast || pl.fast128) && L > 1)
    return fwd_impl(q, k, v, g, beta, u, alpha, p, conv_w, B, H, T, dk, dv, L, chunk, dt, o, S_final,
                    ws + off, workspace_bytes - off, seg_chunks, nullptr, stream, nullptr, nullptr, nullptr,
                    ChainForm::kGelu);
  void* gamma = L > 1 ? ws : nullptr;
  st = prism_nl_gain(v, alpha, p, conv_w, nullptr, B, H, T, dv, L, dt, gamma, stream);
  if (st != PRISM_OK) return st;
  return fwd_impl(q, k, v, g, beta, u, alpha, gamma, conv_w, B, H, T, dk, dv, L, chunk, dt, o, S_final,
                  ws + off, workspace_bytes - off, seg_chunks, nullptr, stream);
}

}  // namespace

extern "C" {

prism_status prism_fwd_nl(const void* q, const void* k, const void* v, const float* g, const float* beta,
                          const void* u, const float* alpha, const void* p, const float* conv_w,
                          int B, int H, int T, int dk, int dv, int L, int chunk, prism_dtype dt,
                          void* o, float* S_final, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return fwd_nl_impl(q, k, v, g, beta, u, alpha, p, conv_w, B, H, T, dk, dv, L, chunk, dt, o, S_final,
                     workspace, workspace_bytes, 0, stream);
}

size_t prism_fwd_nl_seg_workspace_bytes(int B, int H, int T, int dk, int dv, int L, int chunk, prism_dtype dt,
                                        int seg_chunks) {
  Plan pl;
  size_t gb;
  if (seg_chunks <= 0 || make_plan(B, H, T, dk, dv, L, chunk, dt, seg_chunks, &pl) != PRISM_OK ||
      !nl_gamma_bytes(B, H, T, dv, L, dt, &gb))
    return 0;
  return align_up(gb) + pl.total;
}

prism_status prism_fwd_nl_seg(const void* q, const void* k, const void* v, const float* g, const float* beta,
                              const void* u, const float* alpha, const void* p, const float* conv_w,
                              int B, int H, int T, int dk, int dv, int L, int chunk, prism_dtype dt,
                              void* o, float* S_final, void* workspace, size_t workspace_bytes, int seg_chunks,
                              hipStream_t stream) {
  if (seg_chunks <= 0) return PRISM_ERR_INVALID_ARG;
  return fwd_nl_impl(q, k, v, g, beta, u, alpha, p, conv_w, B, H, T, dk, dv, L, chunk, dt, o, S_final,
                     workspace, workspace_bytes, seg_chunks, stream);
}

prism_status prism_nl_gain_pred(const void* v, const float* alpha, const void* W_p, const float* conv_w,
                                const void* conv_in, int B, int H, int T, int dv, int L, prism_dtype dt,
                                void* gamma, hipStream_t stream) {
  if (B <= 0 || H <= 0 || T <= 0) return PRISM_ERR_INVALID_ARG;
  if (dt != PRISM_F32 && dt != PRISM_BF16) return PRISM_ERR_INVALID_ARG;
  if (L < 1 || L > 8) return PRISM_ERR_UNSUPPORTED;
  if (dt != PRISM_BF16 || !(dv == 32 || dv == 64 || dv == 128)) return PRISM_ERR_UNSUPPORTED;
  if (L == 1) return PRISM_OK;
  if (!v || !alpha || !W_p || !conv_w || !gamma) return PRISM_ERR_INVALID_ARG;
  size_t P, bytes;
  if (!mul_ok((size_t)B, (size_t)H, &P) || !nl_gamma_bytes(B, H, T, dv, L, dt, &bytes)) return PRISM_ERR_INVALID_ARG;
  if (P > 65535) return PRISM_ERR_UNSUPPORTED;
  // tokens per workgroup: 4 waves x 4 tiles of 16 at dv = 64, x 2 tiles at 128, else x 1
  const size_t wg_tokens = dv == 64 ? 256 : dv == 128 ? 128 : 64;
  const dim3 grid((unsigned)(((size_t)T + wg_tokens - 1) / wg_tokens), (unsigned)P);
  prism::NlPredArgs a = {};
  a.v = v; a.alpha = alpha; a.W_p = W_p; a.conv_w = conv_w; a.conv_in = conv_in; a.gamma = gamma;
  a.H = H; a.T = T; a.L = L;
  return prism::host::launch_pred(a, dv, grid, false, stream);
}

prism_status prism_fwd_nl_pred(const void* q, const void* k, const void* v, const float* g, const float* beta,
                               const void* u, const float* alpha, const void* W_p, const float* conv_w,
                               int B, int H, int T, int dk, int dv, int L, int chunk, prism_dtype dt,
                               void* o, float* S_final, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  Plan pl;
  prism_status st = make_plan(B, H, T, dk, dv, L, chunk, dt, 0, &pl);
  if (st != PRISM_OK) return st;
  if (L > 1 && (dt != PRISM_BF16 || dv == 16)) return PRISM_ERR_UNSUPPORTED;
  if (!q || !k || !v || !g || !beta || !o || !S_final) return PRISM_ERR_INVALID_ARG;
  if (L > 1 && (!u || !alpha || !W_p || !conv_w)) return PRISM_ERR_INVALID_ARG;
  size_t gb;
  if (!nl_gamma_bytes(B, H, T, dv, L, dt, &gb)) return PRISM_ERR_INVALID_ARG;
  const size_t off = align_up(gb);
  if (!workspace || workspace_bytes < off + pl.total) return PRISM_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  void* gamma = L > 1 ? ws : nullptr;
  st = prism_nl_gain_pred(v, alpha, W_p, conv_w, nullptr, B, H, T, dv, L, dt, gamma, stream);
  if (st != PRISM_OK) return st;
  return fwd_impl(q, k, v, g, beta, u, alpha, gamma, conv_w, B, H, T, dk, dv, L, chunk, dt, o, S_final,
                  ws + off, workspace_bytes - off, 0, nullptr, stream);
}

// ---- the written-correction form -------------------------------------------------------------

size_t prism_fwd_delta_seg_workspace_bytes(int B, int H, int T, int dk, int dv, int L, int chunk, prism_dtype dt,
                                           int seg_chunks) {
  Plan pl;
  size_t gb;
  if (seg_chunks < 0 || make_plan(B, H, T, dk, dv, L, chunk, dt, seg_chunks, &pl) != PRISM_OK ||
      !nl_gamma_bytes(B, H, T, dv, L, dt, &gb))
    return 0;
  return align_up(gb) + pl.total;
}

size_t prism_fwd_delta_workspace_bytes(int B, int H, int T, int dk, int dv, int L, int chunk, prism_dtype dt) {
  return prism_fwd_delta_seg_workspace_bytes(B, H, T, dk, dv, L, chunk, dt, 0);
}

}  // extern "C"

namespace {

prism_status fwd_delta_impl(const void* q, const void* k, const void* v, const float* g, const float* beta,
                            const void* u, const float* alpha, const void* p, const float* conv_w,
                            int B, int H, int T, int dk, int dv, int L, int chunk, prism_dtype dt,
                            void* o, float* S_final, void* workspace, size_t workspace_bytes, int seg_chunks,
                            hipStream_t stream) {
  Plan pl;
  prism_status st = make_plan(B, H, T, dk, dv, L, chunk, dt, seg_chunks, &pl);
  if (st != PRISM_OK) return st;
  if (!q || !k || !v || !g || !beta || !o || !S_final) return PRISM_ERR_INVALID_ARG;
  if (L > 1 && (!u || !alpha || !p || !conv_w)) return PRISM_ERR_INVALID_ARG;
  size_t gb;
  if (!nl_gamma_bytes(B, H, T, dv, L, dt, &gb)) return PRISM_ERR_INVALID_ARG;
  const size_t off = align_up(gb);
  if (!workspace || workspace_bytes < off + pl.total) return PRISM_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  void* fac = L > 1 ? ws : nullptr;
  st = prism_delta_gain(v, p, conv_w, nullptr, B, H, T, dv, L, dt, fac, stream);
  if (st != PRISM_OK) return st;
  return fwd_impl(q, k, v, g, beta, u, alpha, fac, conv_w, B, H, T, dk, dv, L, chunk, dt, o, S_final,
                  ws + off, workspace_bytes - off, seg_chunks, nullptr, stream, nullptr, nullptr, nullptr,
                  ChainForm::kDelta);
}

}  // namespace

extern "C" {

prism_status prism_fwd_delta(const void* q, const void* k, const void* v, const float* g, const float* beta,
                             const void* u, const float* alpha, const void* p, const float* conv_w,
                             int B, int H, int T, int dk, int dv, int L, int chunk, prism_dtype dt,
                             void* o, float* S_final, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  return fwd_delta_impl(q, k, v, g, beta, u, alpha, p, conv_w, B, H, T, dk, dv, L, chunk, dt, o, S_final,
                        workspace, workspace_bytes, 0, stream);
}

prism_status prism_fwd_delta_seg(const void* q, const void* k, const void* v, const float* g, const float* beta,
                                 const void* u, const float* alpha, const void* p, const float* conv_w,
                                 int B, int H, int T, int dk, int dv, int L, int chunk, prism_dtype dt,
                                 void* o, float* S_final, void* workspace, size_t workspace_bytes,
                                 int seg_chunks, hipStream_t stream) {
  if (seg_chunks <= 0) return PRISM_ERR_INVALID_ARG;
  return fwd_delta_impl(q, k, v, g, beta, u, alpha, p, conv_w, B, H, T, dk, dv, L, chunk, dt, o, S_final,
                        workspace, workspace_bytes, seg_chunks, stream);
}

prism_status prism_anchor_predict(const void* v, const float* conv_w, const void* W_p, const void* W_k,
                                  const void* W_b, const void* conv_in, int B, int H, int T, int dk, int dv,
                                  int L, prism_dtype dt, void* gamma, void* u, float* alpha, hipStream_t stream) {
  if (B <= 0 || H <= 0 || T <= 0) return PRISM_ERR_INVALID_ARG;
  if (dt != PRISM_F32 && dt != PRISM_BF16) return PRISM_ERR_INVALID_ARG;
  if (L < 2 || L > 8) return PRISM_ERR_UNSUPPORTED;
  if (dt != PRISM_BF16 || dk != dv || !(dv == 32 || dv == 64 || dv == 128)) return PRISM_ERR_UNSUPPORTED;
  if (!v || !conv_w || !W_p || !W_k || !W_b || !gamma || !u || !alpha) return PRISM_ERR_INVALID_ARG;
  size_t P, bytes;
  if (!mul_ok((size_t)B, (size_t)H, &P) || !nl_gamma_bytes(B, H, T, dv, L, dt, &bytes)) return PRISM_ERR_INVALID_ARG;
  if (P > 65535) return PRISM_ERR_UNSUPPORTED;
  const size_t wg_tokens = dv == 64 ? 256 : 64;  // 4 waves x 16 tokens x tiles per wave
  const dim3 grid((unsigned)(((size_t)T + wg_tokens - 1) / wg_tokens), (unsigned)P);
  prism::NlPredArgs a = {};
  a.v = v; a.W_p = W_p; a.conv_w = conv_w; a.conv_in = conv_in; a.gamma = gamma;
  a.W_k = W_k; a.W_b = W_b; a.u = u; a.alpha_out = alpha;
  a.H = H; a.T = T; a.L = L;
  return prism::host::launch_pred(a, dv, grid, true, stream);
}

}  // extern "C"

namespace {

// Front-end outputs in the workspace of prism_fwd_delta_pred: factors, keys, gates, then
// the forward's own workspace.
struct PredLayout {
  size_t off_u, off_alpha, off_fwd, total;
};

bool pred_layout(int B, int H, int T, int dk, int dv, int L, prism_dtype dt, size_t fwd_bytes, PredLayout* ly) {
  size_t gb, ub, ab, P, pt;
  if (!nl_gamma_bytes(B, H, T, dv, L, dt, &gb) || !nl_gamma_bytes(B, H, T, dk, L, dt, &ub)) return false;
  if (!mul_ok((size_t)B, (size_t)H, &P) || !mul_ok(P, (size_t)T, &pt) || !mul_ok(pt, (size_t)L * 4, &ab))
    return false;
  ly->off_u = align_up(gb);
  ly->off_alpha = align_up(ly->off_u + ub);
  ly->off_fwd = align_up(ly->off_alpha + ab);
  ly->total = ly->off_fwd + fwd_bytes;
  return ly->total >= fwd_bytes;
}

}  // namespace

extern "C" {

size_t prism_fwd_delta_pred_workspace_bytes(int B, int H, int T, int dk, int dv, int L, int chunk, prism_dtype dt) {
  Plan pl;
  PredLayout ly;
  if (L < 2 || dt != PRISM_BF16 || dk != dv || !(dv == 32 || dv == 64 || dv == 128)) return 0;
  if (make_plan(B, H, T, dk, dv, L, chunk, dt, 0, &pl) != PRISM_OK ||
      !pred_layout(B, H, T, dk, dv, L, dt, pl.total, &ly))
    return 0;
  return ly.total;
}

prism_status prism_fwd_delta_pred(const void* q, const void* k, const void* v, const float* g, const float* beta,
                                  const void* W_p, const void* W_k, const void* W_b, const float* conv_w,
                                  int B, int H, int T, int dk, int dv, int L, int chunk, prism_dtype dt,
                                  void* o, float* S_final, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  Plan pl;
  prism_status st = make_plan(B, H, T, dk, dv, L, chunk, dt, 0, &pl);
  if (st != PRISM_OK) return st;
  if (L < 2) return PRISM_ERR_UNSUPPORTED;  // nothing to predict: prism_fwd
  if (dt != PRISM_BF16 || dk != dv || !(dv == 32 || dv == 64 || dv == 128)) return PRISM_ERR_UNSUPPORTED;
  if (!q || !k || !v || !g || !beta || !o || !S_final || !W_p || !W_k || !W_b || !conv_w)
    return PRISM_ERR_INVALID_ARG;
  PredLayout ly;
  if (!pred_layout(B, H, T, dk, dv, L, dt, pl.total, &ly)) return PRISM_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < ly.total) return PRISM_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  void* fac = ws;
  void* uk = ws + ly.off_u;
  float* gates = reinterpret_cast<float*>(ws + ly.off_alpha);
  st = prism_anchor_predict(v, conv_w, W_p, W_k, W_b, nullptr, B, H, T, dk, dv, L, dt, fac, uk, gates, stream);
  if (st != PRISM_OK) return st;
  return fwd_impl(q, k, v, g, beta, uk, gates, fac, conv_w, B, H, T, dk, dv, L, chunk, dt, o, S_final,
                  ws + ly.off_fwd, workspace_bytes - ly.off_fwd, 0, nullptr, stream, nullptr, nullptr, nullptr,
                  ChainForm::kDelta);
}

}  // extern "C"

// ---- the forward without a caller workspace -------------------------------------------------
// The workspace of prism_fwd_noalloc: a file-scope device array, one copy per GPU, held
// until the process ends.  Host code never passes the array's name to a kernel (on the host
// it is only a stand-in for the symbol): it uses the device address that
// hipGetSymbolAddress returns for the current device, looked up once per device.
static __device__ __align__(256) unsigned char scratch[PRISM_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device (null: not looked up)

// The device address of the current device's copy of `scratch`, or null on a HIP error.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

size_t prism_noalloc_scratch_bytes(void) { return PRISM_NOALLOC_SCRATCH_BYTES; }

prism_status prism_fwd_noalloc(const void* q, const void* k, const void* v, const float* g, const float* beta,
                               const void* u, const float* alpha, const void* gamma, const float* conv_w,
                               int B, int H, int T, int dk, int dv, int L, int chunk, prism_dtype dt,
                               void* o, float* S_final, hipStream_t stream) {
  Plan pl;
  prism_status st = make_plan(B, H, T, dk, dv, L, chunk, dt, 0, &pl);
  if (st != PRISM_OK) return st;
  if (!q || !k || !v || !g || !beta || !o || !S_final) return PRISM_ERR_INVALID_ARG;
  if (L > 1 && (!u || !alpha || !gamma || !conv_w)) return PRISM_ERR_INVALID_ARG;
  if (pl.total > (size_t)PRISM_NOALLOC_SCRATCH_BYTES) return PRISM_ERR_WORKSPACE;
  void* ws = scratch_ptr();
  if (ws == nullptr) return PRISM_ERR_HIP;
  // every region of the workspace is written before it is read within one call, so the
  // previous call's contents need no clearing
  return fwd_impl(q, k, v, g, beta, u, alpha, gamma, conv_w, B, H, T, dk, dv, L, chunk, dt, o, S_final,
                  ws, (size_t)PRISM_NOALLOC_SCRATCH_BYTES, 0, nullptr, stream);
}

const char* prism_status_string(prism_status s) {
  switch (s) {
    case PRISM_OK: return "PRISM_OK";
    case PRISM_ERR_INVALID_ARG: return "PRISM_ERR_INVALID_ARG: null pointer, non-positive size or size overflow";
    case PRISM_ERR_UNSUPPORTED: return "PRISM_ERR_UNSUPPORTED: no kernel for this shape / dtype / L / chunk";
    case PRISM_ERR_WORKSPACE: return "PRISM_ERR_WORKSPACE: workspace missing or too small";
    case PRISM_ERR_HIP: return "PRISM_ERR_HIP: a HIP launch failed";
  }
  return "PRISM_ERR_UNKNOWN";
}

const char* prism_version(void) { return "0.1.0"; }

}  // extern "C"
