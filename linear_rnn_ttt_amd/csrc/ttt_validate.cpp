// ttt_validate.cpp -- host-side argument checks of the C ABI: shapes,
// flags, null pointers, sizes, alignment and aliasing, and the fill of the
// kernels' launch arguments.  Plain C++ (no HIP), so argument errors are
// reported the same way with or without a GPU, and the checks build and run
// under the host sanitizers.
#include "ttt_validate.hpp"

#include <cmath>
#include <cstdint>
#include <initializer_list>

namespace tttv {
namespace {

constexpr int32_t kHeadDim = 64;
constexpr int32_t kMlpHidden = 256;
constexpr int32_t kMaxT = 1 << 22;  // tokens per unit

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range span(const void* p, uint64_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + static_cast<uintptr_t>(bytes)};
}

bool overlap(Range a, Range b) {
  if (a.lo == a.hi || b.lo == b.hi || a.lo == 0 || b.lo == 0) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

}  // namespace

ttt_status check_common(const ttt_params* p, uint64_t* elems) {
  if (!p) return TTT_ERR_NULL;
  if (p->io_dtype != TTT_F32 && p->io_dtype != TTT_BF16) return TTT_ERR_ARG;
  if (p->flags & ~static_cast<uint32_t>(TTT_NO_LN | TTT_NO_RESIDUAL)) return TTT_ERR_ARG;
  if (!(p->ln_eps >= 0.0f) || !std::isfinite(p->ln_eps)) return TTT_ERR_ARG;
  if (p->state0_per_batch != 0 && p->state0_per_batch != 1) return TTT_ERR_ARG;
  if (p->B < 1 || p->H < 1 || p->T < 1 || p->d < 1 || p->mini_batch < 1) return TTT_ERR_SHAPE;
  // the kernels address one unit's rows (and its gradient stream) through
  // 32-bit buffer ranges
  if (p->T > kMaxT) return TTT_ERR_SHAPE;
  if (p->d != kHeadDim) return TTT_ERR_UNSUPPORTED;
  const uint64_t units = static_cast<uint64_t>(p->B) * static_cast<uint64_t>(p->H);
  if (units > 0x7fffffffull) return TTT_ERR_SHAPE;  // one workgroup per unit
  const uint64_t tokens = units * static_cast<uint64_t>(p->T);
  if (tokens > (1ull << 40)) return TTT_ERR_SHAPE;
  *elems = tokens * static_cast<uint64_t>(p->d);
  return TTT_OK;
}

SplitLayout split_layout(const ttt_params* p) {
  const uint64_t units = static_cast<uint64_t>(p->B) * p->H;
  const uint64_t tiles = (static_cast<uint64_t>(p->T) + 15) / 16;
  SplitLayout ly;
  ly.stream_offset = (units * 256 + 128 + 255) / 256 * 256;
  ly.total = ly.stream_offset + units * tiles * 6144;
  return ly;
}

void set_split_workspace(const ttt_params* p, void* workspace, tttk::LinearArgs* a) {
  const SplitLayout ly = split_layout(p);
  char* base = static_cast<char*>(workspace);
  a->ws_flags = reinterpret_cast<uint32_t*>(base);
  a->ws_g = reinterpret_cast<uint32_t*>(base + ly.stream_offset);
  a->split = 1;
}

BackwardLayout backward_layout(const ttt_params* p) {
  const uint64_t units = static_cast<uint64_t>(p->B) * p->H;
  const uint64_t tiles = (static_cast<uint64_t>(p->T) + 15) / 16;
  const uint64_t dd4 = static_cast<uint64_t>(kHeadDim) * kHeadDim * 4;
  BackwardLayout ly;
  ly.dw0_offset = units * tiles * dd4;
  ly.dln_offset = ly.dw0_offset + units * dd4;
  ly.front_offset = (ly.dln_offset + units * 2 * kHeadDim * 4 + 255) / 256 * 256;
  // 16-token mini-batches: one record of the front half per unit and tile
  const uint64_t front =
      p->mini_batch == 16 ? units * tiles * static_cast<uint64_t>(tttk::kBwdRecFloats) * 4 : 0;
  ly.total = ly.front_offset + front;
  return ly;
}

ttt_status linear_forward(const ttt_params* p, const void* q, const void* k, const void* v,
                          const float* eta, const float* w0, const float* ln_gamma,
                          const float* ln_beta, void* z, float* w_out, void* workspace,
                          uint64_t workspace_bytes, tttk::LinearArgs* a) {
  uint64_t elems = 0;
  ttt_status st = check_common(p, &elems);
  if (st != TTT_OK) return st;
  const bool ln = !(p->flags & TTT_NO_LN);
  if (!q || !k || !v || !eta || !w0 || !z) return TTT_ERR_NULL;
  if (ln && (!ln_gamma || !ln_beta)) return TTT_ERR_NULL;
  if (p->mini_batch % 16 != 0) return TTT_ERR_UNSUPPORTED;

  const uint64_t es = p->io_dtype == TTT_BF16 ? 2 : 4;
  const uint64_t units = static_cast<uint64_t>(p->B) * p->H;
  const uint64_t dd = static_cast<uint64_t>(kHeadDim) * kHeadDim;
  const Range rq = span(q, elems * es), rk = span(k, elems * es), rv = span(v, elems * es);
  const Range re = span(eta, units * p->T * 4), rz = span(z, elems * es);
  const Range rw0 = span(w0, (p->state0_per_batch ? units : p->H) * dd * 4);
  const Range rg = span(ln ? ln_gamma : nullptr, p->H * 256ull);
  const Range rb = span(ln ? ln_beta : nullptr, p->H * 256ull);
  if (overlap(rz, rq) || overlap(rz, rk) || overlap(rz, rv) || overlap(rz, re) ||
      overlap(rz, rw0) || overlap(rz, rg) || overlap(rz, rb))
    return TTT_ERR_ALIAS;
  const Range rwo = span(w_out, units * dd * 4);
  if (w_out) {
    const bool in_place = p->state0_per_batch == 1 && static_cast<const void*>(w_out) == w0;
    if (overlap(rwo, rq) || overlap(rwo, rk) || overlap(rwo, rv) || overlap(rwo, re) ||
        overlap(rwo, rz) || overlap(rwo, rg) || overlap(rwo, rb) ||
        (!in_place && overlap(rwo, rw0)))
      return TTT_ERR_ALIAS;
  }
  if (workspace) {
    if (workspace_bytes < split_layout(p).total) return TTT_ERR_SHAPE;
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return TTT_ERR_ARG;
    const Range rws = span(workspace, workspace_bytes);
    const Range all[] = {rq, rk, rv, re, rz, rw0, rg, rb, rwo};
    for (const Range& r : all)
      if (overlap(rws, r)) return TTT_ERR_ALIAS;
  }

  a->q = q;
  a->k = k;
  a->v = v;
  a->eta = eta;
  a->w0 = w0;
  a->gamma = ln_gamma;
  a->beta = ln_beta;
  a->z = z;
  a->w_out = w_out;
  a->B = p->B;
  a->H = p->H;
  a->T = p->T;
  a->tiles_per_mb = p->mini_batch / 16;
  a->eps = p->ln_eps;
  a->state0_per_batch = p->state0_per_batch;
  a->ws_g = nullptr;
  a->ws_flags = nullptr;
  a->split = 0;
  a->bases = nullptr;
  return TTT_OK;
}

ttt_status linear_split(const ttt_params* p, const void* q, const void* k, const void* v,
                        const float* eta, const float* w0, const float* ln_gamma,
                        const float* ln_beta, void* z, float* w_out, void* workspace,
                        uint64_t workspace_bytes, tttk::LinearArgs* a) {
  if (!workspace) return TTT_ERR_NULL;
  const ttt_status st = linear_forward(p, q, k, v, eta, w0, ln_gamma, ln_beta, z, w_out,
                                       workspace, workspace_bytes, a);
  if (st != TTT_OK) return st;
  // no in-place resume: the second workgroup of a unit reads the initial
  // state at its own start, which may come after the first has written the
  // final state
  if (w_out && static_cast<const void*>(w_out) == w0) return TTT_ERR_ALIAS;
  set_split_workspace(p, workspace, a);
  return TTT_OK;
}

ttt_status linear_split_noalloc(const ttt_params* p, const void* q, const void* k,
                                const void* v, const float* eta, const float* w0,
                                const float* ln_gamma, const float* ln_beta, void* z,
                                float* w_out, uint64_t scratch_bytes, tttk::LinearArgs* a) {
  const ttt_status st = linear_forward(p, q, k, v, eta, w0, ln_gamma, ln_beta, z, w_out,
                                       nullptr, 0, a);
  if (st != TTT_OK) return st;
  if (w_out && static_cast<const void*>(w_out) == w0) return TTT_ERR_ALIAS;  // as linear_split
  if (split_layout(p).total > scratch_bytes) return TTT_ERR_TOO_LARGE;
  return TTT_OK;
}

ttt_status linear_forward_bases(const ttt_params* p, const void* q, const void* k,
                                const void* v, const float* eta, const float* w0,
                                const float* ln_gamma, const float* ln_beta, void* workspace,
                                tttk::LinearArgs* a) {
  // the workspace stands in for z in the forward's checks (it is checked not
  // to overlap the inputs) and is then replaced by no z at all
  const ttt_status st = linear_forward(p, q, k, v, eta, w0, ln_gamma, ln_beta, workspace,
                                       nullptr, nullptr, 0, a);
  if (st != TTT_OK) return st;
  if (p->mini_batch != 16) return TTT_ERR_UNSUPPORTED;
  a->z = nullptr;
  a->w_out = nullptr;
  a->bases = static_cast<float*>(workspace);
  return TTT_OK;
}

ttt_status linear_forward_save(const ttt_params* p, const void* q, const void* k,
                               const void* v, const float* eta, const float* w0,
                               const float* ln_gamma, const float* ln_beta, void* z,
                               float* w_out, void* workspace, uint64_t workspace_bytes,
                               tttk::LinearArgs* a) {
  const ttt_status st = linear_forward(p, q, k, v, eta, w0, ln_gamma, ln_beta, z, w_out, nullptr,
                                       0, a);
  if (st != TTT_OK) return st;
  if (!workspace) return TTT_ERR_NULL;
  if (p->mini_batch != 16) return TTT_ERR_UNSUPPORTED;
  if (workspace_bytes < backward_layout(p).total) return TTT_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return TTT_ERR_ARG;
  uint64_t elems = 0;
  check_common(p, &elems);
  const uint64_t es = p->io_dtype == TTT_BF16 ? 2 : 4;
  const uint64_t units = static_cast<uint64_t>(p->B) * p->H;
  const uint64_t dd = static_cast<uint64_t>(kHeadDim) * kHeadDim;
  const bool ln = !(p->flags & TTT_NO_LN);
  const Range rws = span(workspace, workspace_bytes);
  const Range all[] = {span(q, elems * es), span(k, elems * es), span(v, elems * es),
                       span(eta, units * p->T * 4),
                       span(w0, (p->state0_per_batch ? units : p->H) * dd * 4),
                       span(ln ? ln_gamma : nullptr, p->H * 256ull),
                       span(ln ? ln_beta : nullptr, p->H * 256ull), span(z, elems * es),
                       span(w_out, units * dd * 4)};
  for (const Range& r : all)
    if (overlap(rws, r)) return TTT_ERR_ALIAS;
  a->bases = static_cast<float*>(workspace);
  return TTT_OK;
}

ttt_status linear_decode(const ttt_params* p, int32_t pos, const void* q, const void* k,
                         const void* v, const float* eta, float* w, float* w_base,
                         const float* ln_gamma, const float* ln_beta, void* z,
                         tttk::DecodeArgs* a) {
  uint64_t elems = 0;
  const ttt_status st = check_common(p, &elems);
  if (st != TTT_OK) return st;
  if (p->T != 1) return TTT_ERR_SHAPE;  // one token per unit
  if (pos < 0 || pos >= p->mini_batch) return TTT_ERR_ARG;
  const bool ln = !(p->flags & TTT_NO_LN);
  if (!q || !k || !v || !eta || !w || !w_base || !z) return TTT_ERR_NULL;
  if (ln && (!ln_gamma || !ln_beta)) return TTT_ERR_NULL;

  const uint64_t es = p->io_dtype == TTT_BF16 ? 2 : 4;
  const uint64_t units = static_cast<uint64_t>(p->B) * p->H;
  const uint64_t dd = static_cast<uint64_t>(kHeadDim) * kHeadDim;
  const Range rq = span(q, elems * es), rk = span(k, elems * es), rv = span(v, elems * es);
  const Range re = span(eta, units * 4), rz = span(z, elems * es);
  const Range rw = span(w, units * dd * 4), rb = span(w_base, units * dd * 4);
  const Range rg = span(ln ? ln_gamma : nullptr, p->H * 256ull);
  const Range rbe = span(ln ? ln_beta : nullptr, p->H * 256ull);
  const Range inputs[] = {rq, rk, rv, re, rg, rbe};
  for (const Range& r : inputs)
    if (overlap(rz, r) || overlap(rw, r) || overlap(rb, r)) return TTT_ERR_ALIAS;
  if (overlap(rz, rw) || overlap(rz, rb) || overlap(rw, rb)) return TTT_ERR_ALIAS;

  a->q = q;
  a->k = k;
  a->v = v;
  a->eta = eta;
  a->w = w;
  a->w_base = w_base;
  a->gamma = ln_gamma;
  a->beta = ln_beta;
  a->z = z;
  a->B = p->B;
  a->H = p->H;
  a->pos = pos;
  a->eps = p->ln_eps;
  return TTT_OK;
}

ttt_status linear_decode_compact(const ttt_params* p, int32_t pos, const void* q,
                                 const void* k, const void* v, const float* eta, float* w_base,
                                 float* hist, const float* ln_gamma, const float* ln_beta,
                                 void* z, tttk::CompactArgs* a) {
  uint64_t elems = 0;
  const ttt_status st = check_common(p, &elems);
  if (st != TTT_OK) return st;
  if (p->T != 1) return TTT_ERR_SHAPE;  // one token per unit
  if (p->mini_batch > 64) return TTT_ERR_UNSUPPORTED;
  if (pos < 0 || pos >= p->mini_batch) return TTT_ERR_ARG;
  const bool ln = !(p->flags & TTT_NO_LN);
  if (!q || !k || !v || !eta || !w_base || !hist || !z) return TTT_ERR_NULL;
  if (ln && (!ln_gamma || !ln_beta)) return TTT_ERR_NULL;

  const uint64_t es = p->io_dtype == TTT_BF16 ? 2 : 4;
  const uint64_t units = static_cast<uint64_t>(p->B) * p->H;
  const uint64_t dd = static_cast<uint64_t>(kHeadDim) * kHeadDim;
  const Range rq = span(q, elems * es), rk = span(k, elems * es), rv = span(v, elems * es);
  const Range re = span(eta, units * 4), rz = span(z, elems * es);
  const Range rw = span(w_base, units * dd * 4);
  const Range rh = span(hist, units * static_cast<uint64_t>(p->mini_batch) * 2 * kHeadDim * 4);
  const Range rg = span(ln ? ln_gamma : nullptr, p->H * 256ull);
  const Range rbe = span(ln ? ln_beta : nullptr, p->H * 256ull);
  const Range inputs[] = {rq, rk, rv, re, rg, rbe};
  for (const Range& r : inputs)
    if (overlap(rz, r) || overlap(rw, r) || overlap(rh, r)) return TTT_ERR_ALIAS;
  if (overlap(rz, rw) || overlap(rz, rh) || overlap(rw, rh)) return TTT_ERR_ALIAS;

  a->q = q;
  a->k = k;
  a->v = v;
  a->eta = eta;
  a->w_base = w_base;
  a->hist = hist;
  a->gamma = ln_gamma;
  a->beta = ln_beta;
  a->z = z;
  a->B = p->B;
  a->H = p->H;
  a->pos = pos;
  a->mb = p->mini_batch;
  a->eps = p->ln_eps;
  return TTT_OK;
}

ttt_status mlp_decode(const ttt_params* p, int32_t hidden, int32_t pos, const void* q,
                      const void* k, const void* v, const float* eta, float* w1, float* b1,
                      float* w2, float* b2, float* w1_base, float* b1_base, float* w2_base,
                      float* b2_base, const float* ln_gamma, const float* ln_beta, void* z,
                      tttk::MlpDecodeArgs* a) {
  uint64_t elems = 0;
  const ttt_status st = check_common(p, &elems);
  if (st != TTT_OK) return st;
  if (p->T != 1) return TTT_ERR_SHAPE;  // one token per unit
  if (hidden < 1) return TTT_ERR_SHAPE;
  if (hidden != kMlpHidden) return TTT_ERR_UNSUPPORTED;
  if (pos < 0 || pos >= p->mini_batch) return TTT_ERR_ARG;
  const bool ln = !(p->flags & TTT_NO_LN);
  float* state[8] = {w1, b1, w2, b2, w1_base, b1_base, w2_base, b2_base};
  if (!q || !k || !v || !eta || !z) return TTT_ERR_NULL;
  for (float* s : state)
    if (!s) return TTT_ERR_NULL;
  if (ln && (!ln_gamma || !ln_beta)) return TTT_ERR_NULL;

  const uint64_t es = p->io_dtype == TTT_BF16 ? 2 : 4;
  const uint64_t units = static_cast<uint64_t>(p->B) * p->H;
  const uint64_t dm = static_cast<uint64_t>(kHeadDim) * hidden;
  const uint64_t sizes[4] = {units * dm * 4, units * hidden * 4ull, units * dm * 4,
                             units * kHeadDim * 4ull};
  const Range rq = span(q, elems * es), rk = span(k, elems * es), rv = span(v, elems * es);
  const Range re = span(eta, units * 4), rz = span(z, elems * es);
  const Range rg = span(ln ? ln_gamma : nullptr, p->H * 256ull);
  const Range rbe = span(ln ? ln_beta : nullptr, p->H * 256ull);
  Range rs[9];
  for (int i = 0; i < 8; ++i) rs[i] = span(state[i], sizes[i % 4]);
  rs[8] = rz;
  const Range inputs[] = {rq, rk, rv, re, rg, rbe};
  for (const Range& w : rs) {
    for (const Range& r : inputs)
      if (overlap(w, r)) return TTT_ERR_ALIAS;
  }
  for (int i = 0; i < 9; ++i)
    for (int j = i + 1; j < 9; ++j)
      if (overlap(rs[i], rs[j])) return TTT_ERR_ALIAS;

  a->q = q;
  a->k = k;
  a->v = v;
  a->eta = eta;
  a->w1 = w1;
  a->b1 = b1;
  a->w2 = w2;
  a->b2 = b2;
  a->w1_base = w1_base;
  a->b1_base = b1_base;
  a->w2_base = w2_base;
  a->b2_base = b2_base;
  a->gamma = ln_gamma;
  a->beta = ln_beta;
  a->z = z;
  a->B = p->B;
  a->H = p->H;
  a->pos = pos;
  a->eps = p->ln_eps;
  return TTT_OK;
}

ttt_status mlp_decode_compact(const ttt_params* p, int32_t hidden, int32_t pos, const void* q,
                              const void* k, const void* v, const float* eta, float* w1_base,
                              float* b1_base, float* w2_base, float* b2_base, float* hist,
                              const float* ln_gamma, const float* ln_beta, void* z,
                              tttk::MlpCompactArgs* a) {
  uint64_t elems = 0;
  const ttt_status st = check_common(p, &elems);
  if (st != TTT_OK) return st;
  if (p->T != 1) return TTT_ERR_SHAPE;  // one token per unit
  if (hidden < 1) return TTT_ERR_SHAPE;
  if (hidden != kMlpHidden || p->mini_batch > 16) return TTT_ERR_UNSUPPORTED;
  if (pos < 0 || pos >= p->mini_batch) return TTT_ERR_ARG;
  const bool ln = !(p->flags & TTT_NO_LN);
  float* state[5] = {w1_base, b1_base, w2_base, b2_base, hist};
  if (!q || !k || !v || !eta || !z) return TTT_ERR_NULL;
  for (float* s : state)
    if (!s) return TTT_ERR_NULL;
  if (ln && (!ln_gamma || !ln_beta)) return TTT_ERR_NULL;

  const uint64_t es = p->io_dtype == TTT_BF16 ? 2 : 4;
  const uint64_t units = static_cast<uint64_t>(p->B) * p->H;
  const uint64_t dm = static_cast<uint64_t>(kHeadDim) * hidden;
  const uint64_t slot = 2ull * kHeadDim + 2ull * hidden;
  const uint64_t sizes[5] = {units * dm * 4, units * hidden * 4ull, units * dm * 4,
                             units * kHeadDim * 4ull,
                             units * static_cast<uint64_t>(p->mini_batch) * slot * 4};
  const Range rq = span(q, elems * es), rk = span(k, elems * es), rv = span(v, elems * es);
  const Range re = span(eta, units * 4), rz = span(z, elems * es);
  const Range rg = span(ln ? ln_gamma : nullptr, p->H * 256ull);
  const Range rbe = span(ln ? ln_beta : nullptr, p->H * 256ull);
  Range rs[6];
  for (int i = 0; i < 5; ++i) rs[i] = span(state[i], sizes[i]);
  rs[5] = rz;
  const Range inputs[] = {rq, rk, rv, re, rg, rbe};
  for (const Range& w : rs) {
    for (const Range& r : inputs)
      if (overlap(w, r)) return TTT_ERR_ALIAS;
  }
  for (int i = 0; i < 6; ++i)
    for (int j = i + 1; j < 6; ++j)
      if (overlap(rs[i], rs[j])) return TTT_ERR_ALIAS;

  a->q = q;
  a->k = k;
  a->v = v;
  a->eta = eta;
  a->w1_base = w1_base;
  a->b1_base = b1_base;
  a->w2_base = w2_base;
  a->b2_base = b2_base;
  a->hist = hist;
  a->gamma = ln_gamma;
  a->beta = ln_beta;
  a->z = z;
  a->B = p->B;
  a->H = p->H;
  a->pos = pos;
  a->mb = p->mini_batch;
  a->eps = p->ln_eps;
  return TTT_OK;
}

ttt_status linear_backward(const ttt_params* p, const void* q, const void* k, const void* v,
                           const float* eta, const float* w0, const float* ln_gamma,
                           const float* ln_beta, const void* dz, const float* dw_final,
                           void* dq, void* dk, void* dv, float* deta, float* dw0,
                           float* dln_gamma, float* dln_beta, void* workspace,
                           uint64_t workspace_bytes, tttk::BackwardArgs* a) {
  if (!p) return TTT_ERR_NULL;
  // TTT_BASES_SAVED is this entry point's own flag; the rest are checked as usual
  const bool saved = (p->flags & TTT_BASES_SAVED) != 0;
  ttt_params pc = *p;
  pc.flags &= ~static_cast<uint32_t>(TTT_BASES_SAVED);
  p = &pc;
  uint64_t elems = 0;
  const ttt_status st = check_common(p, &elems);
  if (st != TTT_OK) return st;
  const bool ln = !(p->flags & TTT_NO_LN);
  if (!q || !k || !v || !eta || !w0 || !dz || !dq || !dk || !dv || !deta || !dw0 || !workspace)
    return TTT_ERR_NULL;
  if (ln && (!ln_gamma || !ln_beta || !dln_gamma || !dln_beta)) return TTT_ERR_NULL;
  if ((dln_gamma == nullptr) != (dln_beta == nullptr)) return TTT_ERR_NULL;
  if (p->mini_batch % 16 != 0 || (saved && p->mini_batch != 16)) return TTT_ERR_UNSUPPORTED;
  const BackwardLayout ly = backward_layout(p);
  if (workspace_bytes < ly.total) return TTT_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return TTT_ERR_ARG;

  const uint64_t es = p->io_dtype == TTT_BF16 ? 2 : 4;
  const uint64_t units = static_cast<uint64_t>(p->B) * p->H;
  const uint64_t dd = static_cast<uint64_t>(kHeadDim) * kHeadDim;
  const uint64_t w0_bytes = (p->state0_per_batch ? units : p->H) * dd * 4;
  const Range inputs[] = {
      span(q, elems * es), span(k, elems * es), span(v, elems * es),
      span(eta, units * p->T * 4), span(w0, w0_bytes),
      span(ln ? ln_gamma : nullptr, p->H * 256ull), span(ln ? ln_beta : nullptr, p->H * 256ull),
      span(dz, elems * es), span(dw_final, units * dd * 4)};
  const Range outputs[] = {
      span(dq, elems * es), span(dk, elems * es), span(dv, elems * es),
      span(deta, units * p->T * 4), span(dw0, w0_bytes), span(dln_gamma, p->H * 256ull),
      span(dln_beta, p->H * 256ull), span(workspace, workspace_bytes)};
  const int n_out = sizeof(outputs) / sizeof(outputs[0]);
  for (int i = 0; i < n_out; ++i) {
    for (const Range& r : inputs)
      if (overlap(outputs[i], r)) return TTT_ERR_ALIAS;
    for (int j = i + 1; j < n_out; ++j)
      if (overlap(outputs[i], outputs[j])) return TTT_ERR_ALIAS;
  }

  a->q = q;
  a->k = k;
  a->v = v;
  a->eta = eta;
  a->w0 = w0;
  a->gamma = ln_gamma;
  a->beta = ln_beta;
  a->dz = dz;
  a->dw_final = dw_final;
  a->dq = dq;
  a->dk = dk;
  a->dv = dv;
  a->deta = deta;
  a->dw0 = dw0;
  a->dgamma = dln_gamma;
  a->dbeta = dln_beta;
  char* base = static_cast<char*>(workspace);
  a->ws_base = reinterpret_cast<float*>(base);
  a->ws_dw0 = reinterpret_cast<float*>(base + ly.dw0_offset);
  a->ws_dln = reinterpret_cast<float*>(base + ly.dln_offset);
  a->ws_front = p->mini_batch == 16 ? reinterpret_cast<float*>(base + ly.front_offset) : nullptr;
  a->B = p->B;
  a->H = p->H;
  a->T = p->T;
  a->tiles_per_mb = p->mini_batch / 16;
  a->eps = p->ln_eps;
  a->state0_per_batch = p->state0_per_batch;
  a->bases_saved = saved ? 1 : 0;
  return TTT_OK;
}

ttt_status mlp_forward(const ttt_params* p, int32_t hidden, const void* q, const void* k,
                       const void* v, const float* eta, const float* w1_0, const float* b1_0,
                       const float* w2_0, const float* b2_0, const float* ln_gamma,
                       const float* ln_beta, void* z, float* w1_out, float* b1_out,
                       float* w2_out, float* b2_out, tttk::MlpArgs* a) {
  uint64_t elems = 0;
  ttt_status st = check_common(p, &elems);
  if (st != TTT_OK) return st;
  if (hidden < 1) return TTT_ERR_SHAPE;
  const bool ln = !(p->flags & TTT_NO_LN);
  if (!q || !k || !v || !eta || !w1_0 || !b1_0 || !w2_0 || !b2_0 || !z) return TTT_ERR_NULL;
  if (ln && (!ln_gamma || !ln_beta)) return TTT_ERR_NULL;
  const int n_out = (w1_out != nullptr) + (b1_out != nullptr) + (w2_out != nullptr) +
                    (b2_out != nullptr);
  if (n_out != 0 && n_out != 4) return TTT_ERR_NULL;
  if (hidden != kMlpHidden || p->mini_batch != 16) return TTT_ERR_UNSUPPORTED;

  const uint64_t es = p->io_dtype == TTT_BF16 ? 2 : 4;
  const uint64_t units = static_cast<uint64_t>(p->B) * p->H;
  const uint64_t s0 = p->state0_per_batch ? units : static_cast<uint64_t>(p->H);
  const uint64_t dm = static_cast<uint64_t>(kHeadDim) * hidden;
  const Range rq = span(q, elems * es), rk = span(k, elems * es), rv = span(v, elems * es);
  const Range re = span(eta, units * p->T * 4), rz = span(z, elems * es);
  const Range rin[4] = {span(w1_0, s0 * dm * 4), span(b1_0, s0 * hidden * 4),
                        span(w2_0, s0 * dm * 4), span(b2_0, s0 * kHeadDim * 4)};
  const Range rg = span(ln ? ln_gamma : nullptr, p->H * 256ull);
  const Range rb = span(ln ? ln_beta : nullptr, p->H * 256ull);
  const Range inputs[] = {rq, rk, rv, re, rg, rb, rin[0], rin[1], rin[2], rin[3]};
  for (const Range& r : inputs)
    if (overlap(rz, r)) return TTT_ERR_ALIAS;
  if (n_out == 4) {
    float* outs[4] = {w1_out, b1_out, w2_out, b2_out};
    const void* ins[4] = {w1_0, b1_0, w2_0, b2_0};
    const uint64_t sizes[4] = {units * dm * 4, units * hidden * 4ull, units * dm * 4,
                               units * kHeadDim * 4ull};
    Range ro[4];
    for (int i = 0; i < 4; ++i) ro[i] = span(outs[i], sizes[i]);
    for (int i = 0; i < 4; ++i) {
      if (overlap(ro[i], rq) || overlap(ro[i], rk) || overlap(ro[i], rv) ||
          overlap(ro[i], re) || overlap(ro[i], rz) || overlap(ro[i], rg) || overlap(ro[i], rb))
        return TTT_ERR_ALIAS;
      for (int j = 0; j < 4; ++j) {
        if (j != i && overlap(ro[i], ro[j])) return TTT_ERR_ALIAS;
        const bool in_place = i == j && p->state0_per_batch == 1 &&
                              static_cast<const void*>(outs[i]) == ins[i];
        if (!in_place && overlap(ro[i], rin[j])) return TTT_ERR_ALIAS;
      }
    }
  }

  a->q = q;
  a->k = k;
  a->v = v;
  a->eta = eta;
  a->w1 = w1_0;
  a->b1 = b1_0;
  a->w2 = w2_0;
  a->b2 = b2_0;
  a->gamma = ln_gamma;
  a->beta = ln_beta;
  a->z = z;
  a->w1_out = w1_out;
  a->b1_out = b1_out;
  a->w2_out = w2_out;
  a->b2_out = b2_out;
  a->B = p->B;
  a->H = p->H;
  a->T = p->T;
  a->eps = p->ln_eps;
  a->state0_per_batch = p->state0_per_batch;
  return TTT_OK;
}

uint64_t mlp_backward_unit_floats(const ttt_params* p) {
  const uint64_t n = (static_cast<uint64_t>(p->T) + 15) / 16;
  return (n + 1) * tttk::MLP_BWD_STATE_FLOATS + tttk::MLP_BWD_TILE_FLOATS;
}

uint64_t mlp_backward_workspace_bytes(const ttt_params* p) {
  const uint64_t units = static_cast<uint64_t>(p->B) * p->H;
  return (units * mlp_backward_unit_floats(p) * 4 + 255) / 256 * 256;
}

ttt_status mlp_backward(const ttt_params* p, int32_t hidden, const void* q, const void* k,
                        const void* v, const float* eta, const float* w1_0, const float* b1_0,
                        const float* w2_0, const float* b2_0, const float* ln_gamma,
                        const float* ln_beta, const void* dz, const float* dw1_final,
                        const float* db1_final, const float* dw2_final, const float* db2_final,
                        void* dq, void* dk, void* dv, float* deta, float* dw1, float* db1,
                        float* dw2, float* db2, float* dln_gamma, float* dln_beta,
                        void* workspace, uint64_t workspace_bytes, tttk::MlpBackwardArgs* a) {
  uint64_t elems = 0;
  const ttt_status st = check_common(p, &elems);
  if (st != TTT_OK) return st;
  if (hidden < 1) return TTT_ERR_SHAPE;
  const bool ln = !(p->flags & TTT_NO_LN);
  if (!q || !k || !v || !eta || !w1_0 || !b1_0 || !w2_0 || !b2_0 || !dz || !dq || !dk || !dv ||
      !deta || !dw1 || !db1 || !dw2 || !db2 || !workspace)
    return TTT_ERR_NULL;
  if (ln && (!ln_gamma || !ln_beta || !dln_gamma || !dln_beta)) return TTT_ERR_NULL;
  if ((dln_gamma == nullptr) != (dln_beta == nullptr)) return TTT_ERR_NULL;
  const int n_fin = (dw1_final != nullptr) + (db1_final != nullptr) + (dw2_final != nullptr) +
                    (db2_final != nullptr);
  if (n_fin != 0 && n_fin != 4) return TTT_ERR_NULL;
  if (hidden != kMlpHidden || p->mini_batch != 16) return TTT_ERR_UNSUPPORTED;
  if (workspace_bytes < mlp_backward_workspace_bytes(p)) return TTT_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return TTT_ERR_ARG;

  const uint64_t es = p->io_dtype == TTT_BF16 ? 2 : 4;
  const uint64_t units = static_cast<uint64_t>(p->B) * p->H;
  const uint64_t s0 = p->state0_per_batch ? units : static_cast<uint64_t>(p->H);
  const uint64_t dm = static_cast<uint64_t>(kHeadDim) * hidden;
  const uint64_t ssz[4] = {dm * 4, static_cast<uint64_t>(hidden) * 4, dm * 4, kHeadDim * 4ull};
  const Range inputs[] = {
      span(q, elems * es), span(k, elems * es), span(v, elems * es),
      span(eta, units * p->T * 4), span(w1_0, s0 * ssz[0]), span(b1_0, s0 * ssz[1]),
      span(w2_0, s0 * ssz[2]), span(b2_0, s0 * ssz[3]),
      span(ln ? ln_gamma : nullptr, p->H * 256ull), span(ln ? ln_beta : nullptr, p->H * 256ull),
      span(dz, elems * es), span(dw1_final, units * ssz[0]), span(db1_final, units * ssz[1]),
      span(dw2_final, units * ssz[2]), span(db2_final, units * ssz[3])};
  const Range outputs[] = {
      span(dq, elems * es), span(dk, elems * es), span(dv, elems * es),
      span(deta, units * p->T * 4), span(dw1, s0 * ssz[0]), span(db1, s0 * ssz[1]),
      span(dw2, s0 * ssz[2]), span(db2, s0 * ssz[3]), span(dln_gamma, p->H * 256ull),
      span(dln_beta, p->H * 256ull), span(workspace, workspace_bytes)};
  const int n_out = sizeof(outputs) / sizeof(outputs[0]);
  for (int i = 0; i < n_out; ++i) {
    for (const Range& r : inputs)
      if (overlap(outputs[i], r)) return TTT_ERR_ALIAS;
    for (int j = i + 1; j < n_out; ++j)
      if (overlap(outputs[i], outputs[j])) return TTT_ERR_ALIAS;
  }

  a->q = q;
  a->k = k;
  a->v = v;
  a->eta = eta;
  a->w1 = w1_0;
  a->b1 = b1_0;
  a->w2 = w2_0;
  a->b2 = b2_0;
  a->gamma = ln_gamma;
  a->beta = ln_beta;
  a->dz = dz;
  a->dw1_final = dw1_final;
  a->db1_final = db1_final;
  a->dw2_final = dw2_final;
  a->db2_final = db2_final;
  a->dq = dq;
  a->dk = dk;
  a->dv = dv;
  a->deta = deta;
  a->dw1 = dw1;
  a->db1 = db1;
  a->dw2 = dw2;
  a->db2 = db2;
  a->dgamma = dln_gamma;
  a->dbeta = dln_beta;
  a->ws = static_cast<float*>(workspace);
  a->unit_floats = mlp_backward_unit_floats(p);
  a->B = p->B;
  a->H = p->H;
  a->T = p->T;
  a->eps = p->ln_eps;
  a->state0_per_batch = p->state0_per_batch;
  return TTT_OK;
}

ttt_status input_projection(const ttt_params* p, int32_t d_model, const void* x,
                            const void* w_in, const float* b_eta, float eta_base, void* q,
                            void* k, void* v, float* eta, tttk::InputArgs* a) {
  uint64_t elems = 0;
  const ttt_status st = check_common(p, &elems);
  if (st != TTT_OK) return st;
  if (!x || !w_in || !b_eta || !q || !k || !v || !eta) return TTT_ERR_NULL;
  if (d_model < 1) return TTT_ERR_SHAPE;
  if (p->io_dtype != TTT_BF16 || d_model % 64 != 0) return TTT_ERR_UNSUPPORTED;
  if (!(eta_base > 0.0f) || !std::isfinite(eta_base)) return TTT_ERR_ARG;
  for (const void* ptr : {x, w_in, static_cast<const void*>(q), static_cast<const void*>(k),
                          static_cast<const void*>(v)})
    if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0) return TTT_ERR_ARG;
  const uint64_t tokens = static_cast<uint64_t>(p->B) * p->T;
  if (tokens > (1ull << 30)) return TTT_ERR_SHAPE;   // the kernel indexes rows with int
  const uint64_t n_out = 3ull * p->H * kHeadDim + p->H;
  const Range inputs[] = {span(x, tokens * d_model * 2), span(w_in, n_out * d_model * 2),
                          span(b_eta, p->H * 4ull)};
  const Range outputs[] = {span(q, elems * 2), span(k, elems * 2), span(v, elems * 2),
                           span(eta, tokens * p->H * 4ull)};
  const int n_o = sizeof(outputs) / sizeof(outputs[0]);
  for (int i = 0; i < n_o; ++i) {
    for (const Range& r : inputs)
      if (overlap(outputs[i], r)) return TTT_ERR_ALIAS;
    for (int j2 = i + 1; j2 < n_o; ++j2)
      if (overlap(outputs[i], outputs[j2])) return TTT_ERR_ALIAS;
  }
  a->x = x;
  a->w = w_in;
  a->b_eta = b_eta;
  a->q = q;
  a->k = k;
  a->v = v;
  a->eta = eta;
  a->B = p->B;
  a->T = p->T;
  a->D = d_model;
  a->H = p->H;
  a->eta_base = eta_base;
  return TTT_OK;
}

}  // namespace tttv
