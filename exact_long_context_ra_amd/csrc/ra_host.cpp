// Host side of the C ABI declared in include/ra.h: argument validation, the
// token-to-device layouts, the virtual-ring step planner and kernel timing.
//
// Layouts ("Ring Flash Attention" README function list; guijiagi.com Ring
// Attention article, sections on the detailed flow and on striped ring
// attention; Striped Attention abstract on briefgpt.xyz):
//   contiguous  rank r owns positions [r*L, (r+1)*L)                 L = S/N
//   zigzag      rank r owns chunks r and 2N-1-r of size C = S/(2N), in that order
//   stripe      rank r owns positions r, r+N, r+2N, ...
// Ring schedule (same article, detailed flow): at step s the rank works on the
// block of rank (r - s) mod N.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "ra.h"
#include "ra_internal.h"

using namespace ra;

namespace {

thread_local char g_err[1024] = "";

ra_status fail(ra_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

#define RA_CHECK(cond, status, ...) \
  do {                              \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

#define RA_HIP(expr)                                                                               \
  do {                                                                                             \
    hipError_t e_ = (expr);                                                                        \
    if (e_ != hipSuccess) return fail(RA_ERR_HIP, "%s failed: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

constexpr int64_t kMaxPos = 0x7fffffffLL;

// ---- timing -------------------------------------------------------------------------------

struct Timing {
  bool on = false;
  int cap = 0;
  int n = 0;
  std::vector<hipEvent_t> ev0, ev1;
  std::vector<int32_t> kid, step;
};
thread_local Timing g_timing;

template <class F>
hipError_t timed(KernelId id, int step, hipStream_t s, F&& f) {
  Timing& t = g_timing;
  if (!t.on || t.n >= t.cap) return f();
  const int i = t.n;
  hipError_t e = hipEventRecord(t.ev0[i], s);
  if (e != hipSuccess) return e;
  e = f();
  if (e != hipSuccess) return e;
  e = hipEventRecord(t.ev1[i], s);
  if (e != hipSuccess) return e;
  t.kid[i] = id;
  t.step[i] = step;
  t.n = i + 1;
  return hipSuccess;
}

// ---- validation ---------------------------------------------------------------------------

ra_status check_problem(const ra_problem* p) {
  RA_CHECK(p != nullptr, RA_ERR_INVALID_ARG, "problem is NULL");
  RA_CHECK(p->batch >= 1 && p->heads >= 1, RA_ERR_INVALID_ARG, "batch (%d) and heads (%d) must be >= 1", p->batch,
           p->heads);
  RA_CHECK(p->dtype == RA_DTYPE_F32 || p->dtype == RA_DTYPE_BF16, RA_ERR_INVALID_ARG, "unknown dtype %d",
           (int)p->dtype);
  RA_CHECK(p->head_dim == 64 || p->head_dim == 128, RA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)",
           p->head_dim);
  RA_CHECK(p->seq_len >= 0 && p->seq_len <= kMaxPos, RA_ERR_INVALID_ARG, "seq_len %lld out of range",
           (long long)p->seq_len);
  RA_CHECK(isfinite(p->softmax_scale), RA_ERR_INVALID_ARG, "softmax_scale is not finite");
  RA_CHECK(p->num_seqs >= 0, RA_ERR_INVALID_ARG, "num_seqs must be >= 0");
  if (p->num_seqs > 0) {
    RA_CHECK(p->cu_seqlens != nullptr, RA_ERR_INVALID_ARG, "num_seqs > 0 but cu_seqlens is NULL");
    RA_CHECK(p->batch == 1, RA_ERR_INVALID_ARG, "cu_seqlens requires batch == 1 (got %d)", p->batch);
    if (p->cu_seqlens_host) {
      const int32_t* cu = p->cu_seqlens_host;
      RA_CHECK(cu[0] == 0, RA_ERR_INVALID_ARG, "cu_seqlens[0] must be 0");
      for (int i = 0; i < p->num_seqs; ++i)
        RA_CHECK(cu[i + 1] >= cu[i], RA_ERR_INVALID_ARG, "cu_seqlens must be non-decreasing (index %d)", i + 1);
      RA_CHECK(cu[p->num_seqs] == p->seq_len, RA_ERR_INVALID_ARG, "cu_seqlens[num_seqs]=%d != seq_len=%lld",
               cu[p->num_seqs], (long long)p->seq_len);
    }
  } else {
    RA_CHECK(p->cu_seqlens == nullptr, RA_ERR_INVALID_ARG, "cu_seqlens given but num_seqs == 0");
  }
  return RA_OK;
}

size_t elem_size(ra_dtype d) { return d == RA_DTYPE_BF16 ? 2 : 4; }

// Results and accumulators (out, dQ, dK, dV and their bf16 copies): the kernels
// address them with 64-bit pointer arithmetic, so their slices may be of any
// size.
ra_status check_out_tensor(const char* name, const ra_tensor& t, size_t esz, bool need) {
  if (!need) return RA_OK;
  RA_CHECK(t.ptr != nullptr, RA_ERR_INVALID_ARG, "%s: NULL pointer", name);
  RA_CHECK(((uintptr_t)t.ptr & 15) == 0, RA_ERR_INVALID_ARG, "%s: pointer not 16-byte aligned", name);
  RA_CHECK(t.stride_b >= 0 && t.stride_t >= 0 && t.stride_h >= 0, RA_ERR_INVALID_ARG, "%s: negative stride", name);
  const int64_t b16 = 16 / (int64_t)esz;  // elements per 16 bytes
  RA_CHECK(t.stride_b % b16 == 0 && t.stride_t % b16 == 0 && t.stride_h % b16 == 0, RA_ERR_INVALID_ARG,
           "%s: strides must keep rows 16-byte aligned", name);
  return RA_OK;
}

// Operands the kernels read through buffer descriptors (q, k, v, dout).
ra_status check_tensor(const char* name, const ra_tensor& t, size_t esz, int64_t rows, bool need) {
  if (!need) return RA_OK;
  ra_status st = check_out_tensor(name, t, esz, need);
  if (st != RA_OK) return st;
  // One (batch, head) slice is addressed with 32-bit byte offsets, and reads go
  // up to 256 rows past its end (those reads return zeros).
  RA_CHECK((rows + 256) * t.stride_t * (int64_t)esz + 512 * (int64_t)esz < (int64_t(1) << 31), RA_ERR_UNSUPPORTED,
           "%s: a (batch, head) slice spans more than 2 GiB", name);
  return RA_OK;
}

ra_status check_ptr(const char* name, const void* p) {
  RA_CHECK(p != nullptr, RA_ERR_INVALID_ARG, "%s: NULL pointer", name);
  RA_CHECK(((uintptr_t)p & 3) == 0, RA_ERR_INVALID_ARG, "%s: pointer not 4-byte aligned", name);
  return RA_OK;
}

int64_t pos_at(const ra_posmap& m, int64_t a) {
  if (a < m.seg[0].len) return m.seg[0].begin + a * m.seg[0].stride;
  return m.seg[1].begin + (a - m.seg[0].len) * m.seg[1].stride;
}

ra_status check_posmap(const char* name, const ra_posmap& m, int64_t len, int64_t seq_len) {
  RA_CHECK(m.nseg == 1 || m.nseg == 2, RA_ERR_INVALID_ARG, "%s: nseg must be 1 or 2 (got %d)", name, m.nseg);
  int64_t total = 0;
  int64_t prev_last = -1;
  for (int i = 0; i < m.nseg; ++i) {
    const ra_seg& s = m.seg[i];
    RA_CHECK(s.len >= 0 && s.stride >= 1 && s.begin >= 0, RA_ERR_INVALID_ARG,
             "%s: segment %d needs len >= 0, stride >= 1, begin >= 0", name, i);
    if (s.len > 0) {
      const int64_t last = s.begin + (s.len - 1) * s.stride;
      RA_CHECK(last < seq_len && last <= kMaxPos, RA_ERR_INVALID_ARG, "%s: segment %d exceeds seq_len", name, i);
      RA_CHECK(s.begin > prev_last, RA_ERR_INVALID_ARG, "%s: positions must be strictly increasing", name);
      prev_last = last;
    }
    total += s.len;
  }
  RA_CHECK(total == len, RA_ERR_INVALID_ARG, "%s: segment lengths sum to %lld, expected %lld", name,
           (long long)total, (long long)len);
  return RA_OK;
}

DMap to_dmap(const ra_posmap& m) {
  DMap d{};
  d.nseg = m.nseg;
  d.s0 = DSeg{(int32_t)m.seg[0].begin, (int32_t)m.seg[0].stride, (int32_t)m.seg[0].len};
  if (m.nseg == 2)
    d.s1 = DSeg{(int32_t)m.seg[1].begin, (int32_t)m.seg[1].stride, (int32_t)m.seg[1].len};
  else
    d.s1 = DSeg{0, 1, 0};
  d.total = d.s0.len + d.s1.len;
  return d;
}

MaskSpec mask_of(const ra_problem* p) {
  MaskSpec m{};
  m.causal = p->causal ? 1 : 0;
  m.nseq = p->num_seqs;
  m.cu = p->cu_seqlens;
  return m;
}

float scale_of(const ra_problem* p) {
  return p->softmax_scale > 0.f ? p->softmax_scale : 1.0f / sqrtf((float)p->head_dim);
}

Tensor4 rd(const ra_tensor& t) { return Tensor4{t.ptr, t.stride_b, t.stride_t, t.stride_h}; }
Tensor4W wr(const ra_tensor& t) { return Tensor4W{t.ptr, t.stride_b, t.stride_t, t.stride_h}; }
Tensor4 offset_rd(const ra_tensor& t, int64_t elems, size_t esz) {
  return Tensor4{(const char*)t.ptr + elems * (int64_t)esz, t.stride_b, t.stride_t, t.stride_h};
}
Tensor4W offset_wr(const ra_tensor& t, int64_t elems, size_t esz) {
  return Tensor4W{(char*)t.ptr + elems * (int64_t)esz, t.stride_b, t.stride_t, t.stride_h};
}

// ---- layouts ------------------------------------------------------------------------------

ra_status make_posmap(ra_layout layout, int64_t S, int32_t N, int32_t r, ra_posmap* out) {
  RA_CHECK(N >= 1, RA_ERR_INVALID_ARG, "world must be >= 1");
  RA_CHECK(r >= 0 && r < N, RA_ERR_INVALID_ARG, "rank %d out of range [0, %d)", r, N);
  RA_CHECK(S >= 0 && S <= kMaxPos, RA_ERR_INVALID_ARG, "seq_len out of range");
  ra_posmap m{};
  switch (layout) {
    case RA_LAYOUT_CONTIGUOUS: {
      RA_CHECK(S % N == 0, RA_ERR_INVALID_ARG, "contiguous: seq_len %lld not divisible by world %d", (long long)S, N);
      const int64_t L = S / N;
      m.nseg = 1;
      m.seg[0] = ra_seg{r * L, 1, L};
      break;
    }
    case RA_LAYOUT_ZIGZAG: {
      RA_CHECK(S % (2 * (int64_t)N) == 0, RA_ERR_INVALID_ARG, "zigzag: seq_len %lld not divisible by 2*world",
               (long long)S);
      const int64_t C = S / (2 * (int64_t)N);
      m.nseg = 2;
      m.seg[0] = ra_seg{r * C, 1, C};
      m.seg[1] = ra_seg{(2 * (int64_t)N - 1 - r) * C, 1, C};
      break;
    }
    case RA_LAYOUT_STRIPE: {
      RA_CHECK(S % N == 0, RA_ERR_INVALID_ARG, "stripe: seq_len %lld not divisible by world %d", (long long)S, N);
      m.nseg = 1;
      m.seg[0] = ra_seg{r, N, S / N};
      break;
    }
    case RA_LAYOUT_ZIGZAG_VARLEN:
    case RA_LAYOUT_STRIPE_VARLEN:
      return fail(RA_ERR_UNSUPPORTED, "layout %d has one posmap per sequence (see ra_layout_positions_cu)",
                  (int)layout);
    default:
      return fail(RA_ERR_INVALID_ARG, "unknown layout %d", (int)layout);
  }
  *out = m;
  return RA_OK;
}

// First local index with position >= P (len if none); last with position <= P (-1 if none).
int64_t h_first_ge(const ra_posmap& m, int64_t P) {
  int64_t off = 0;
  for (int i = 0; i < m.nseg; ++i) {
    const ra_seg& s = m.seg[i];
    if (s.len > 0) {
      const int64_t last = s.begin + (s.len - 1) * s.stride;
      if (last >= P) return off + (P <= s.begin ? 0 : (P - s.begin + s.stride - 1) / s.stride);
    }
    off += s.len;
  }
  return off;
}
int64_t h_last_le(const ra_posmap& m, int64_t P) {
  int64_t off = 0;
  int64_t best = -1;
  for (int i = 0; i < m.nseg; ++i) {
    const ra_seg& s = m.seg[i];
    if (s.len > 0 && P >= s.begin) {
      int64_t k = (P - s.begin) / s.stride;
      if (k > s.len - 1) k = s.len - 1;
      best = off + k;
    }
    off += s.len;
  }
  return best;
}

// Does any (query, key) pair of these posmaps survive the mask?
bool step_has_pairs(const ra_problem* p, const ra_posmap& qm, int64_t lq, const ra_posmap& km, int64_t lk) {
  if (lq == 0 || lk == 0) return false;
  const int64_t qmax = pos_at(qm, lq - 1);
  const int64_t kmin = pos_at(km, 0);
  if (p->num_seqs > 0 && p->cu_seqlens_host) {
    const int32_t* cu = p->cu_seqlens_host;
    for (int s = 0; s < p->num_seqs; ++s) {
      const int64_t a = cu[s], e = cu[s + 1] - 1;
      if (a > e) continue;
      const int64_t qi = h_last_le(qm, e), ki = h_first_ge(km, a);
      if (qi < 0 || ki >= lk) continue;
      const int64_t qp = pos_at(qm, qi), kp = pos_at(km, ki);
      if (qp < a || kp > e) continue;
      if (!p->causal || kp <= qp) return true;
    }
    return false;
  }
  return !p->causal || kmin <= qmax;
}

int32_t ceil_div(int64_t a, int64_t b) { return (int32_t)((a + b - 1) / b); }

}  // namespace

// ============================================================================================
// C ABI
// ============================================================================================

extern "C" {

const char* ra_status_str(ra_status s) {
  switch (s) {
    case RA_OK: return "RA_OK";
    case RA_ERR_INVALID_ARG: return "RA_ERR_INVALID_ARG";
    case RA_ERR_UNSUPPORTED: return "RA_ERR_UNSUPPORTED";
    case RA_ERR_HIP: return "RA_ERR_HIP";
    case RA_ERR_WORKSPACE: return "RA_ERR_WORKSPACE";
  }
  return "RA_ERR_UNKNOWN";
}

const char* ra_last_error(void) { return g_err; }

int ra_abi_version(void) { return RA_ABI_VERSION; }

const char* ra_kernel_name(int32_t id) {
  switch (id) {
    case K_FWD: return "block_fwd";
    case K_BWD: return "block_bwd_dkdv";
    case K_BWD_DQ: return "block_bwd_dq";
    case K_BWD_DQ_DS: return "block_bwd_dq_ds";
    case K_MERGE: return "lse_merge";
    case K_PREP: return "bwd_preprocess";
    case K_CAST: return "cast_bf16";
    case K_ZERO: return "zero";
  }
  return "unknown";
}

ra_status ra_layout_posmap(ra_layout layout, int64_t seq_len, int32_t world, int32_t rank, ra_posmap* out) {
  RA_CHECK(out != nullptr, RA_ERR_INVALID_ARG, "out is NULL");
  return make_posmap(layout, seq_len, world, rank, out);
}

ra_status ra_layout_positions(ra_layout layout, int64_t seq_len, int32_t world, int32_t rank, int64_t* host_pos_out) {
  RA_CHECK(host_pos_out != nullptr, RA_ERR_INVALID_ARG, "host_pos_out is NULL");
  ra_posmap m;
  ra_status st = make_posmap(layout, seq_len, world, rank, &m);
  if (st != RA_OK) return st;
  int64_t a = 0;
  for (int i = 0; i < m.nseg; ++i)
    for (int64_t j = 0; j < m.seg[i].len; ++j) host_pos_out[a++] = m.seg[i].begin + j * m.seg[i].stride;
  return RA_OK;
}

ra_status ra_layout_positions_cu(ra_layout layout, const int32_t* cu_host, int32_t num_seqs, int32_t world,
                                 int32_t rank, int64_t* host_pos_out) {
  RA_CHECK(host_pos_out != nullptr, RA_ERR_INVALID_ARG, "host_pos_out is NULL");
  RA_CHECK(cu_host != nullptr && num_seqs >= 1, RA_ERR_INVALID_ARG, "cu_host with num_seqs >= 1 required");
  RA_CHECK(cu_host[0] == 0, RA_ERR_INVALID_ARG, "cu_seqlens[0] must be 0");
  for (int i = 0; i < num_seqs; ++i)
    RA_CHECK(cu_host[i + 1] >= cu_host[i], RA_ERR_INVALID_ARG, "cu_seqlens must be non-decreasing");
  if (layout != RA_LAYOUT_ZIGZAG_VARLEN && layout != RA_LAYOUT_STRIPE_VARLEN)
    return ra_layout_positions(layout, cu_host[num_seqs], world, rank, host_pos_out);
  RA_CHECK(world >= 1 && rank >= 0 && rank < world, RA_ERR_INVALID_ARG, "rank %d / world %d out of range", rank,
           world);
  const ra_layout base = layout == RA_LAYOUT_ZIGZAG_VARLEN ? RA_LAYOUT_ZIGZAG : RA_LAYOUT_STRIPE;
  int64_t a = 0;
  for (int i = 0; i < num_seqs; ++i) {
    ra_posmap m;
    ra_status st = make_posmap(base, (int64_t)cu_host[i + 1] - cu_host[i], world, rank, &m);
    if (st != RA_OK) {
      char why[sizeof(g_err)];
      snprintf(why, sizeof(why), "%s", g_err);
      return fail(st, "sequence %d: %s", i, why);
    }
    for (int k = 0; k < m.nseg; ++k)
      for (int64_t j = 0; j < m.seg[k].len; ++j)
        host_pos_out[a++] = cu_host[i] + m.seg[k].begin + j * m.seg[k].stride;
  }
  return RA_OK;
}

ra_status ra_timing_begin(int32_t capacity) {
  RA_CHECK(capacity >= 1 && capacity <= RA_MAX_TIMED_LAUNCHES, RA_ERR_INVALID_ARG, "capacity %d out of range",
           capacity);
  Timing& t = g_timing;
  while ((int)t.ev0.size() < capacity) {
    hipEvent_t a, b;
    RA_HIP(hipEventCreate(&a));
    RA_HIP(hipEventCreate(&b));
    t.ev0.push_back(a);
    t.ev1.push_back(b);
  }
  t.kid.assign(capacity, -1);
  t.step.assign(capacity, -1);
  t.cap = capacity;
  t.n = 0;
  t.on = true;
  return RA_OK;
}

ra_status ra_timing_end(ra_launch_time* out, int32_t capacity, int32_t* n_out) {
  Timing& t = g_timing;
  RA_CHECK(t.on, RA_ERR_INVALID_ARG, "timing was not started");
  RA_CHECK(n_out != nullptr, RA_ERR_INVALID_ARG, "n_out is NULL");
  RA_CHECK(out != nullptr || capacity == 0, RA_ERR_INVALID_ARG, "out is NULL");
  t.on = false;
  const int n = t.n < capacity ? t.n : capacity;
  if (t.n > 0) RA_HIP(hipEventSynchronize(t.ev1[t.n - 1]));
  for (int i = 0; i < n; ++i) {
    float ms = 0.f;
    RA_HIP(hipEventElapsedTime(&ms, t.ev0[i], t.ev1[i]));
    out[i] = ra_launch_time{t.kid[i], t.step[i], ms};
  }
  *n_out = n;
  t.n = 0;
  return RA_OK;
}

ra_status ra_cast_f32_to_bf16(const float* src, void* dst, int64_t n, void* stream) {
  RA_CHECK(n >= 0, RA_ERR_INVALID_ARG, "n must be >= 0");
  if (n == 0) return RA_OK;
  RA_CHECK(src != nullptr && dst != nullptr, RA_ERR_INVALID_ARG, "NULL pointer");
  RA_HIP(timed(K_CAST, -1, (hipStream_t)stream, [&] { return launch_cast(src, dst, n, (hipStream_t)stream); }));
  return RA_OK;
}

ra_status ra_block_attn_fwd(const ra_problem* prob, ra_tensor q, int64_t lq, ra_posmap qmap, ra_tensor k, ra_tensor v,
                            int64_t lk, ra_posmap kmap, ra_tensor out_b, float* lse_b, void* stream) {
  ra_status st = check_problem(prob);
  if (st != RA_OK) return st;
  RA_CHECK(lq >= 0 && lq <= kMaxPos && lk >= 0 && lk <= kMaxPos, RA_ERR_INVALID_ARG, "lq/lk out of range");
  if (lq == 0) return RA_OK;
  const size_t esz = elem_size(prob->dtype);
  if ((st = check_tensor("q", q, esz, lq, true)) != RA_OK) return st;
  if ((st = check_tensor("k", k, esz, lk, lk > 0)) != RA_OK) return st;
  if ((st = check_tensor("v", v, esz, lk, lk > 0)) != RA_OK) return st;
  if ((st = check_out_tensor("out_b", out_b, 4, true)) != RA_OK) return st;
  if ((st = check_ptr("lse_b", lse_b)) != RA_OK) return st;
  if ((st = check_posmap("qmap", qmap, lq, prob->seq_len)) != RA_OK) return st;
  if (lk > 0 && (st = check_posmap("kmap", kmap, lk, prob->seq_len)) != RA_OK) return st;

  FwdArgs a{};
  a.q = rd(q);
  a.k = rd(k);
  a.v = rd(v);
  a.out = wr(out_b);
  a.lse = lse_b;
  a.out_lowp = Tensor4W{nullptr, 0, 0, 0};
  a.batch = prob->batch;
  a.heads = prob->heads;
  a.lq = (int32_t)lq;
  a.lse_sh = lq;
  a.lk = (int32_t)lk;
  a.qmap = to_dmap(qmap);
  if (lk > 0) a.kmap = to_dmap(kmap);
  a.mask = mask_of(prob);
  a.scale_log2 = scale_of(prob) * 1.4426950408889634f;
  a.mode = FWD_STORE;
  a.n_qtiles = ceil_div(lq, FWD_BQ);
  const bool bf16 = prob->dtype == RA_DTYPE_BF16;
  hipStream_t s = (hipStream_t)stream;
  RA_HIP(timed(K_FWD, -1, s, [&] { return launch_fwd(a, prob->head_dim, bf16, s); }));
  return RA_OK;
}

ra_status ra_lse_merge(const ra_problem* prob, int64_t lq, ra_tensor out, float* lse, ra_tensor out_b,
                       const float* lse_b, void* stream) {
  ra_status st = check_problem(prob);
  if (st != RA_OK) return st;
  RA_CHECK(lq >= 0 && lq <= kMaxPos, RA_ERR_INVALID_ARG, "lq out of range");
  if (lq == 0) return RA_OK;
  if ((st = check_out_tensor("out", out, 4, true)) != RA_OK) return st;
  if ((st = check_out_tensor("out_b", out_b, 4, true)) != RA_OK) return st;
  if ((st = check_ptr("lse", lse)) != RA_OK) return st;
  if ((st = check_ptr("lse_b", lse_b)) != RA_OK) return st;
  MergeArgs a{};
  a.out = wr(out);
  a.lse = lse;
  a.out_b = rd(out_b);
  a.lse_b = lse_b;
  a.batch = prob->batch;
  a.heads = prob->heads;
  a.lq = (int32_t)lq;
  a.dim = prob->head_dim;
  hipStream_t s = (hipStream_t)stream;
  RA_HIP(timed(K_MERGE, -1, s, [&] { return launch_merge(a, s); }));
  return RA_OK;
}

ra_status ra_bwd_preprocess(const ra_problem* prob, int64_t lq, ra_tensor out, ra_tensor dout, float* delta,
                            void* stream) {
  ra_status st = check_problem(prob);
  if (st != RA_OK) return st;
  RA_CHECK(lq >= 0 && lq <= kMaxPos, RA_ERR_INVALID_ARG, "lq out of range");
  if (lq == 0) return RA_OK;
  if ((st = check_out_tensor("out", out, 4, true)) != RA_OK) return st;
  if ((st = check_tensor("dout", dout, elem_size(prob->dtype), lq, true)) != RA_OK) return st;
  if ((st = check_ptr("delta", delta)) != RA_OK) return st;
  PrepArgs a{};
  a.out = rd(out);
  a.dout = rd(dout);
  a.delta = delta;
  a.batch = prob->batch;
  a.heads = prob->heads;
  a.lq = (int32_t)lq;
  a.dim = prob->head_dim;
  hipStream_t s = (hipStream_t)stream;
  const bool bf16 = prob->dtype == RA_DTYPE_BF16;
  RA_HIP(timed(K_PREP, -1, s, [&] { return launch_prep(a, bf16, s); }));
  return RA_OK;
}

// One backward block step: bf16 runs the dK/dV kernel and then dQ, from the dS
// it stored when a.dsT is set, else by recomputing S and dP; fp32 runs the fused kernel.
static ra_status launch_bwd_step(const BwdArgs& a, int head_dim, bool bf16, int step, hipStream_t s) {
  if (bf16) {
    RA_HIP(timed(K_BWD, step, s, [&] { return launch_bwd_dkdv(a, head_dim, s); }));
    if (a.dsT)
      RA_HIP(timed(K_BWD_DQ_DS, step, s, [&] { return launch_bwd_dq_ds(a, head_dim, s); }));
    else
      RA_HIP(timed(K_BWD_DQ, step, s, [&] { return launch_bwd_dq(a, head_dim, s); }));
  } else {
    RA_HIP(timed(K_BWD, step, s, [&] { return launch_bwd_fused_f32(a, head_dim, s); }));
  }
  return RA_OK;
}

static ra_status bwd_args(const ra_problem* prob, ra_tensor q, int64_t lq, const ra_posmap& qmap, Tensor4 k,
                          Tensor4 v, int64_t lk, const ra_posmap& kmap, ra_tensor dout, const float* lse,
                          const float* delta, Tensor4W dq, Tensor4W dk, Tensor4W dv, BwdArgs* out) {
  BwdArgs a{};
  a.q = rd(q);
  a.k = k;
  a.v = v;
  a.dout = rd(dout);
  a.lse = lse;
  a.delta = delta;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.batch = prob->batch;
  a.heads = prob->heads;
  a.lq = (int32_t)lq;
  a.lse_sh = lq;
  a.lk = (int32_t)lk;
  a.qmap = to_dmap(qmap);
  a.kmap = to_dmap(kmap);
  a.mask = mask_of(prob);
  a.scale = scale_of(prob);
  a.scale_log2 = a.scale * 1.4426950408889634f;
  a.n_ktiles = ceil_div(lk, BWD_BK);
  a.n_qtiles = ceil_div(lq, FWD_BQ);
  *out = a;
  return RA_OK;
}

ra_status ra_block_attn_bwd(const ra_problem* prob, ra_tensor q, int64_t lq, ra_posmap qmap, ra_tensor k, ra_tensor v,
                            int64_t lk, ra_posmap kmap, ra_tensor dout, const float* lse, const float* delta,
                            ra_tensor dq_acc, ra_tensor dk_acc, ra_tensor dv_acc, void* stream) {
  ra_status st = check_problem(prob);
  if (st != RA_OK) return st;
  RA_CHECK(lq >= 0 && lq <= kMaxPos && lk >= 0 && lk <= kMaxPos, RA_ERR_INVALID_ARG, "lq/lk out of range");
  if (lq == 0 || lk == 0) return RA_OK;
  const size_t esz = elem_size(prob->dtype);
  if ((st = check_tensor("q", q, esz, lq, true)) != RA_OK) return st;
  if ((st = check_tensor("k", k, esz, lk, true)) != RA_OK) return st;
  if ((st = check_tensor("v", v, esz, lk, true)) != RA_OK) return st;
  if ((st = check_tensor("dout", dout, esz, lq, true)) != RA_OK) return st;
  if ((st = check_out_tensor("dq_acc", dq_acc, 4, true)) != RA_OK) return st;
  if ((st = check_out_tensor("dk_acc", dk_acc, 4, true)) != RA_OK) return st;
  if ((st = check_out_tensor("dv_acc", dv_acc, 4, true)) != RA_OK) return st;
  if ((st = check_ptr("lse", lse)) != RA_OK) return st;
  if ((st = check_ptr("delta", delta)) != RA_OK) return st;
  if ((st = check_posmap("qmap", qmap, lq, prob->seq_len)) != RA_OK) return st;
  if ((st = check_posmap("kmap", kmap, lk, prob->seq_len)) != RA_OK) return st;
  BwdArgs a;
  bwd_args(prob, q, lq, qmap, rd(k), rd(v), lk, kmap, dout, lse, delta, wr(dq_acc), wr(dk_acc), wr(dv_acc), &a);
  hipStream_t s = (hipStream_t)stream;
  const bool bf16 = prob->dtype == RA_DTYPE_BF16;
  return launch_bwd_step(a, prob->head_dim, bf16, -1, s);
}

// ---- virtual ring -------------------------------------------------------------------------

static bool per_seq_layout(ra_layout l) { return l == RA_LAYOUT_ZIGZAG_VARLEN || l == RA_LAYOUT_STRIPE_VARLEN; }
static ra_layout base_layout(ra_layout l) {
  return l == RA_LAYOUT_ZIGZAG_VARLEN ? RA_LAYOUT_ZIGZAG : l == RA_LAYOUT_STRIPE_VARLEN ? RA_LAYOUT_STRIPE : l;
}

// One independent ring: the whole problem for the plain layouts; one packed
// sequence for the per-sequence layouts (sequences never attend to each other,
// and each one's local tokens are the run of rows [row0, row0 + L) of every
// rank's buffers).  `prob` is the piece's own problem: for a sequence, its
// length as seq_len and no cu_seqlens (one sequence, positions from 0).
struct Piece {
  ra_problem prob;
  int64_t row0, L;
};

static ra_status ring_pieces(const ra_problem* prob, ra_layout layout, int32_t world, std::vector<Piece>* out) {
  out->clear();
  if (!per_seq_layout(layout)) {
    ra_posmap m;
    ra_status st = make_posmap(layout, prob->seq_len, world, 0, &m);
    if (st != RA_OK) return st;
    out->push_back(Piece{*prob, 0, prob->seq_len / world});
    return RA_OK;
  }
  RA_CHECK(prob->num_seqs > 0 && prob->cu_seqlens != nullptr && prob->cu_seqlens_host != nullptr,
           RA_ERR_INVALID_ARG, "layout %d needs cu_seqlens and its host copy", (int)layout);
  const int64_t unit = layout == RA_LAYOUT_ZIGZAG_VARLEN ? 2 * (int64_t)world : world;
  const int32_t* cu = prob->cu_seqlens_host;
  for (int i = 0; i < prob->num_seqs; ++i) {
    const int64_t n = (int64_t)cu[i + 1] - cu[i];
    RA_CHECK(n % unit == 0, RA_ERR_INVALID_ARG, "sequence %d: length %lld not divisible by %lld", i, (long long)n,
             (long long)unit);
    if (n == 0) continue;
    Piece pc{*prob, cu[i] / world, n / world};
    pc.prob.seq_len = n;
    pc.prob.cu_seqlens = nullptr;
    pc.prob.cu_seqlens_host = nullptr;
    pc.prob.num_seqs = 0;
    out->push_back(pc);
  }
  return RA_OK;
}

static ra_status ring_common(const ra_problem* prob, ra_layout layout, int32_t world, int32_t rank, int64_t* L,
                             std::vector<Piece>* pieces) {
  ra_status st = check_problem(prob);
  if (st != RA_OK) return st;
  RA_CHECK(world >= 1, RA_ERR_INVALID_ARG, "world must be >= 1");
  RA_CHECK(rank >= 0 && rank < world, RA_ERR_INVALID_ARG, "rank %d out of range [0, %d)", rank, world);
  RA_CHECK(layout >= RA_LAYOUT_CONTIGUOUS && layout <= RA_LAYOUT_STRIPE_VARLEN, RA_ERR_INVALID_ARG,
           "unknown layout %d", (int)layout);
  if ((st = ring_pieces(prob, layout, world, pieces)) != RA_OK) return st;
  *L = prob->seq_len / world;
  return RA_OK;
}

// rows further down a [b, rows, h, d] tensor
static ra_tensor shift_rows(const ra_tensor& t, int64_t rows, size_t esz) {
  ra_tensor u = t;
  if (t.ptr) u.ptr = (char*)t.ptr + rows * t.stride_t * (int64_t)esz;
  return u;
}

// Independent rings (the sequences of a per-sequence layout) run concurrently
// on a few side streams, forked from and joined back into the caller's stream
// with events: one sequence's launches are small, and one after another they
// leave most of the GPU idle.  Each host thread keeps its own streams and
// events per device (default priority, non-blocking), created on first use and
// kept until the process ends.
constexpr int kSideStreams = 4;
struct SidePool {
  bool ready = false;
  hipStream_t st[kSideStreams];
  hipEvent_t fork, join[kSideStreams];
};

static ra_status side_pool(SidePool** out) {
  static thread_local std::vector<SidePool> pools;
  int dev = 0;
  RA_HIP(hipGetDevice(&dev));
  if ((int)pools.size() <= dev) pools.resize(dev + 1);
  SidePool& p = pools[dev];
  if (!p.ready) {
    for (int k = 0; k < kSideStreams; ++k) {
      RA_HIP(hipStreamCreateWithFlags(&p.st[k], hipStreamNonBlocking));
      RA_HIP(hipEventCreateWithFlags(&p.join[k], hipEventDisableTiming));
    }
    RA_HIP(hipEventCreateWithFlags(&p.fork, hipEventDisableTiming));
    p.ready = true;
  }
  *out = &p;
  return RA_OK;
}

// Side stream of every piece: longest first onto the least-loaded stream (work
// taken as L^2), over `nstreams` streams.
static std::vector<int> assign_pieces(const std::vector<Piece>& pieces, int nstreams) {
  std::vector<int> order(pieces.size()), where(pieces.size(), 0);
  for (size_t i = 0; i < order.size(); ++i) order[i] = (int)i;
  std::sort(order.begin(), order.end(), [&](int x, int y) { return pieces[x].L > pieces[y].L; });
  std::vector<double> load(nstreams, 0.0);
  for (int i : order) {
    int best = 0;
    for (int k = 1; k < nstreams; ++k)
      if (load[k] < load[best]) best = k;
    where[i] = best;
    load[best] += (double)pieces[i].L * (double)pieces[i].L;
  }
  return where;
}

static ra_status fork_streams(SidePool* p, int n, hipStream_t s) {
  RA_HIP(hipEventRecord(p->fork, s));
  for (int k = 0; k < n; ++k) RA_HIP(hipStreamWaitEvent(p->st[k], p->fork, 0));
  return RA_OK;
}

static ra_status join_streams(SidePool* p, int n, hipStream_t s) {
  for (int k = 0; k < n; ++k) {
    RA_HIP(hipEventRecord(p->join[k], p->st[k]));
    RA_HIP(hipStreamWaitEvent(s, p->join[k], 0));
  }
  return RA_OK;
}

// The forward ring of one piece: rows [row0, row0 + pc.L) of the local buffers;
// lse rows at lse + row0 with head stride lse_sh.
static ra_status ring_fwd_piece(const Piece& pc, ra_layout layout, int32_t world, int32_t rank, ra_tensor q_local,
                                ra_tensor k_ring, ra_tensor v_ring, int64_t stride_rank, ra_tensor out, float* lse,
                                int64_t lse_sh, ra_tensor out_lowp, hipStream_t s) {
  const ra_problem* prob = &pc.prob;
  const int64_t L = pc.L;
  const size_t esz = elem_size(prob->dtype);
  q_local = shift_rows(q_local, pc.row0, esz);
  k_ring = shift_rows(k_ring, pc.row0, esz);
  v_ring = shift_rows(v_ring, pc.row0, esz);
  out = shift_rows(out, pc.row0, 4);
  out_lowp = shift_rows(out_lowp, pc.row0, esz);

  ra_posmap qmap;
  make_posmap(layout, prob->seq_len, world, rank, &qmap);
  std::vector<int> steps;
  std::vector<ra_posmap> kmaps(world);
  for (int st = 0; st < world; ++st) {
    const int src = ((rank - st) % world + world) % world;
    make_posmap(layout, prob->seq_len, world, src, &kmaps[st]);
    if (step_has_pairs(prob, qmap, L, kmaps[st], L)) steps.push_back(st);
  }
  if (steps.empty()) steps.push_back(0);  // still writes (0, -inf) rows

  FwdArgs a{};
  a.q = rd(q_local);
  a.out = wr(out);
  a.lse = lse + pc.row0;
  a.lse_sh = lse_sh;
  a.batch = prob->batch;
  a.heads = prob->heads;
  a.lq = (int32_t)L;
  a.lk = (int32_t)L;
  a.qmap = to_dmap(qmap);
  a.mask = mask_of(prob);
  a.scale_log2 = scale_of(prob) * 1.4426950408889634f;
  a.n_qtiles = ceil_div(L, FWD_BQ);
  const bool bf16 = prob->dtype == RA_DTYPE_BF16;
  for (size_t i = 0; i < steps.size(); ++i) {
    const int step = steps[i];
    const int src = ((rank - step) % world + world) % world;
    a.k = offset_rd(k_ring, src * stride_rank, esz);
    a.v = offset_rd(v_ring, src * stride_rank, esz);
    a.kmap = to_dmap(kmaps[step]);
    a.mode = (i == 0) ? FWD_STORE : FWD_MERGE;
    a.out_lowp = (i + 1 == steps.size()) ? wr(out_lowp) : Tensor4W{nullptr, 0, 0, 0};
    RA_HIP(timed(K_FWD, step, s, [&] { return launch_fwd(a, prob->head_dim, bf16, s); }));
  }
  return RA_OK;
}

// Ring schedule of every piece of a per-sequence layout: its posmaps and, per
// step, whether any pair is visible (a piece without any visible pair still
// runs step 0, which writes its (0, -inf) rows).
struct PiecePlan {
  ra_posmap qmap;
  std::vector<ra_posmap> kmap;  // per step
  std::vector<char> active;     // per step
  int first = -1, last = -1;    // first and last active step
  bool forced = false;          // no visible pair at all: step 0 only writes (0, -inf)
};

static std::vector<PiecePlan> plan_pieces(const std::vector<Piece>& pieces, ra_layout lay, int32_t world,
                                          int32_t rank) {
  std::vector<PiecePlan> plans(pieces.size());
  for (size_t i = 0; i < pieces.size(); ++i) {
    const Piece& pc = pieces[i];
    PiecePlan& pl = plans[i];
    make_posmap(lay, pc.prob.seq_len, world, rank, &pl.qmap);
    pl.kmap.resize(world);
    pl.active.assign(world, 0);
    for (int st = 0; st < world; ++st) {
      const int src = ((rank - st) % world + world) % world;
      make_posmap(lay, pc.prob.seq_len, world, src, &pl.kmap[st]);
      pl.active[st] = step_has_pairs(&pc.prob, pl.qmap, pc.L, pl.kmap[st], pc.L) ? 1 : 0;
    }
    for (int st = 0; st < world; ++st)
      if (pl.active[st]) {
        if (pl.first < 0) pl.first = st;
        pl.last = st;
      }
    if (pl.first < 0) {
      pl.active[0] = 1;
      pl.first = pl.last = 0;
      pl.forced = true;
    }
  }
  return plans;
}

// First local query row of a piece, rounded down to a multiple of 16, from
// which its rows can see a key of this step's block: under the causal mask a
// row sees nothing before the block's first key position, and positions grow
// with the row.  The forward and dQ launches start there (a per-sequence
// zigzag ring's first chunk sees no key after step 0, so its rows would
// otherwise fill, and straddle, whole row tiles for nothing).
static int32_t first_seeing_row(const Piece& pc, const ra_posmap& qmap, const ra_posmap& kmap) {
  if (!pc.prob.causal || pc.prob.num_seqs > 0 || pc.L == 0) return 0;
  const int64_t qa = std::min<int64_t>(h_first_ge(qmap, pos_at(kmap, 0)), pc.L - 1);
  return (int32_t)(qa / 16 * 16);
}

// The pieces active at `step`, longest first, in groups of at most kMaxPieces.
// Workgroups are dispatched roughly in id order and a longer piece has the
// longer-running workgroups, so putting it first keeps them off the end of the
// launch.
static std::vector<std::vector<int>> step_groups(const std::vector<Piece>& pieces,
                                                 const std::vector<PiecePlan>& plans, int step,
                                                 bool skip_forced = false) {
  std::vector<int> order(plans.size());
  for (size_t i = 0; i < order.size(); ++i) order[i] = (int)i;
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return pieces[x].L > pieces[y].L; });
  std::vector<std::vector<int>> groups;
  for (int i : order) {
    if (!plans[i].active[step] || (skip_forced && plans[i].forced)) continue;
    if (groups.empty() || (int)groups.back().size() == kMaxPieces) groups.emplace_back();
    groups.back().push_back(i);
  }
  return groups;
}

// bf16 forward of a per-sequence layout: per ring step, one launch over every
// sequence that has visible pairs at that step (a piece table in the kernel
// arguments), instead of one small launch per sequence.
static ra_status ring_fwd_grouped(const std::vector<Piece>& pieces, ra_layout layout, int32_t world, int32_t rank,
                                  ra_tensor q_local, ra_tensor k_ring, ra_tensor v_ring, int64_t stride_rank,
                                  ra_tensor out, float* lse, int64_t L, ra_tensor out_lowp, hipStream_t s) {
  const ra_problem* prob = &pieces[0].prob;
  const size_t esz = elem_size(prob->dtype);
  const std::vector<PiecePlan> plans = plan_pieces(pieces, base_layout(layout), world, rank);
  FwdArgs base{};
  base.q = rd(q_local);
  base.out = wr(out);
  base.lse = lse;
  base.lse_sh = L;
  base.out_lowp = wr(out_lowp);
  base.batch = prob->batch;
  base.heads = prob->heads;
  base.lq = base.lk = (int32_t)L;
  base.mask = mask_of(prob);
  base.scale_log2 = scale_of(prob) * 1.4426950408889634f;
  for (int step = 0; step < world; ++step) {
    const int src = ((rank - step) % world + world) % world;
    for (const std::vector<int>& grp : step_groups(pieces, plans, step)) {
      FwdArgs a = base;
      a.k = offset_rd(k_ring, src * stride_rank, esz);
      a.v = offset_rd(v_ring, src * stride_rank, esz);
      a.g.n = (int32_t)grp.size();
      for (size_t j = 0; j < grp.size(); ++j) {
        const int i = grp[j];
        a.g.row0[j] = (int32_t)pieces[i].row0;
        a.g.len[j] = (int32_t)pieces[i].L;
        const bool merge = step != plans[i].first, lowp = step == plans[i].last && out_lowp.ptr;
        a.g.flags[j] = (merge ? PIECE_MERGE : 0) | (lowp ? PIECE_LOWP : 0);
        // rows that see no key are left out only where a merge leaves them as
        // they are (not on the step that first stores them or writes the copy)
        a.g.qoff[j] = merge && !lowp ? first_seeing_row(pieces[i], plans[i].qmap, plans[i].kmap[step]) : 0;
        a.g.qmap[j] = to_dmap(plans[i].qmap);
        a.g.kmap[j] = to_dmap(plans[i].kmap[step]);
      }
      RA_HIP(timed(K_FWD, step, s, [&] { return launch_fwd(a, prob->head_dim, true, s); }));
    }
  }
  return RA_OK;
}

ra_status ra_ring_fwd(const ra_problem* prob, ra_layout layout, int32_t world, int32_t rank, ra_tensor q_local,
                      ra_tensor k_ring, ra_tensor v_ring, int64_t stride_rank, ra_tensor out, float* lse,
                      ra_tensor out_lowp, void* stream) {
  int64_t L = 0;
  std::vector<Piece> pieces;
  ra_status st = ring_common(prob, layout, world, rank, &L, &pieces);
  if (st != RA_OK) return st;
  if (L == 0) return RA_OK;
  const size_t esz = elem_size(prob->dtype);
  if ((st = check_tensor("q_local", q_local, esz, L, true)) != RA_OK) return st;
  if ((st = check_tensor("k_ring", k_ring, esz, L, true)) != RA_OK) return st;
  if ((st = check_tensor("v_ring", v_ring, esz, L, true)) != RA_OK) return st;
  if ((st = check_out_tensor("out", out, 4, true)) != RA_OK) return st;
  if ((st = check_out_tensor("out_lowp", out_lowp, esz, out_lowp.ptr != nullptr)) != RA_OK) return st;
  if ((st = check_ptr("lse", lse)) != RA_OK) return st;
  RA_CHECK(stride_rank >= 0 && stride_rank % (int64_t)(16 / esz) == 0, RA_ERR_INVALID_ARG,
           "stride_rank must be >= 0 and keep 16-byte alignment");
  hipStream_t s = (hipStream_t)stream;
  if (pieces.size() == 1)
    return ring_fwd_piece(pieces[0], base_layout(layout), world, rank, q_local, k_ring, v_ring, stride_rank, out,
                          lse, L, out_lowp, s);
  if (prob->dtype == RA_DTYPE_BF16)
    return ring_fwd_grouped(pieces, layout, world, rank, q_local, k_ring, v_ring, stride_rank, out, lse, L,
                            out_lowp, s);
  // fp32 (the parity path): one ring per sequence, the rings on side streams
  SidePool* pool = nullptr;
  if ((st = side_pool(&pool)) != RA_OK) return st;
  const int ns = (int)std::min<size_t>(kSideStreams, pieces.size());
  const std::vector<int> where = assign_pieces(pieces, ns);
  if ((st = fork_streams(pool, ns, s)) != RA_OK) return st;
  for (size_t i = 0; i < pieces.size() && st == RA_OK; ++i)
    st = ring_fwd_piece(pieces[i], base_layout(layout), world, rank, q_local, k_ring, v_ring, stride_rank, out, lse,
                        L, out_lowp, pool->st[where[i]]);
  const ra_status sj = join_streams(pool, ns, s);
  return st != RA_OK ? st : sj;
}

// Workspace of ra_ring_bwd: delta [b, h, L] fp32 (rounded up to 256 bytes), then
// for bf16 the dS^T buffer of one piece at a time: per (b, h) a blocked
// [keys][query rows] slice of round_up(Lp, 128) keys (whole dK/dV key tiles) by
// ds_ld = round_up(Lp, 128) rows (whole dQ row tiles), bf16, for the largest
// piece length Lp.
static int64_t ds_ld_of(int64_t L) { return (L + FWD_BQ - 1) / FWD_BQ * FWD_BQ; }

// dS^T bytes of a piece of Lp local rows, or 0 where the stored-dS path does
// not apply (fp32, or one (b, h) slice beyond the 32-bit byte offsets of a
// buffer descriptor: Lp above 46336).
static size_t ds_bytes(const ra_problem* prob, int64_t Lp) {
  if (prob->dtype != RA_DTYPE_BF16 || Lp == 0) return 0;
  const int64_t slice = (Lp + BWD_BK - 1) / BWD_BK * BWD_BK * ds_ld_of(Lp) * 2;
  if (slice >= ((int64_t)1 << 32)) return 0;
  return (size_t)prob->batch * prob->heads * (size_t)slice;
}

// dS^T of every piece side by side, for a grouped backward (0 unless every
// piece fits the stored-dS path).
static size_t ds_bytes_sum(const std::vector<Piece>& pieces) {
  size_t sum = 0;
  for (const Piece& pc : pieces) {
    const size_t b = ds_bytes(&pc.prob, pc.L);
    if (b == 0) return 0;
    sum += b;
  }
  return sum;
}


size_t ra_ring_workspace_min_bytes(const ra_problem* prob, ra_layout layout, int32_t world) {
  int64_t L = 0;
  std::vector<Piece> pieces;
  if (ring_common(prob, layout, world, 0, &L, &pieces) != RA_OK) return 0;
  const size_t bytes = (size_t)prob->batch * prob->heads * L * sizeof(float);
  return (bytes + 255) & ~(size_t)255;
}

// A block's keys can also go through the stored-dS path a chunk at a time:
// for each chunk of keys the dK/dV kernel writes that chunk's dS^T and the dQ
// kernel adds its dS K into dQ, so the dS^T buffer holds one chunk (dK/dV of a
// key depend on its own chunk only; dQ sums the chunks in turn).  That bounds
// the buffer for any block length, which keeps long blocks (a (b, h) slice of
// 4 GiB or more) and smaller workspaces on the five-product path instead of
// recomputing S and dP for dQ.  Chunks are whole dK/dV key tiles and at least
// kMinDsChunk keys: shorter ones leave the dQ workgroups too little work.
constexpr int64_t kMinDsChunk = 1024;
// dS^T that the default workspace provides for a block whose whole dS^T does
// not fit 4 GiB (b, h) slices: chunks of at most this many bytes in all.
constexpr size_t kDefaultDsChunkBytes = (size_t)32 << 30;

static int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

// dS^T bytes per key of a block with lq query rows, over all (b, h) slices.
static int64_t ds_bytes_per_key(const ra_problem* p, int64_t lq) {
  return (int64_t)p->batch * p->heads * ds_ld_of(lq) * 2;
}

// Keys per dS^T chunk of a block of lq rows x lk keys with `avail` bytes for
// dS^T: the whole (tile-padded) block when it fits, else the largest multiple
// of the key tile that fits and keeps one (b, h) slice under 4 GiB; 0 (dQ
// recomputes S and dP) when that is under kMinDsChunk keys, and for fp32.
static int64_t ds_chunk_keys(const ra_problem* p, int64_t lq, int64_t lk, size_t avail) {
  if (p->dtype != RA_DTYPE_BF16 || lq == 0 || lk == 0) return 0;
  const int64_t full = round_up(lk, BWD_BK);
  const int64_t slice_cap = ((((int64_t)1 << 32) - 1) / (ds_ld_of(lq) * 2)) / BWD_BK * BWD_BK;
  int64_t kc = std::min<int64_t>((int64_t)(avail / (size_t)ds_bytes_per_key(p, lq)), slice_cap);
  kc = kc / BWD_BK * BWD_BK;
  if (kc >= full) return full;
  return kc >= kMinDsChunk ? kc : 0;
}

// dS^T bytes of the default workspace for one block: the whole block when its
// (b, h) slices stay under 4 GiB, else chunks within kDefaultDsChunkBytes.
static size_t ds_default_bytes(const ra_problem* p, int64_t lq, int64_t lk) {
  if (p->dtype != RA_DTYPE_BF16 || lq == 0 || lk == 0) return 0;
  const int64_t full = round_up(lk, BWD_BK);
  if (full * ds_ld_of(lq) * 2 < ((int64_t)1 << 32)) return (size_t)(full * ds_bytes_per_key(p, lq));
  return (size_t)(ds_chunk_keys(p, lq, lk, kDefaultDsChunkBytes) * ds_bytes_per_key(p, lq));
}

// Local indices [c0, c0 + n) of a posmap as a posmap of their own.
static ra_posmap sub_posmap(const ra_posmap& m, int64_t c0, int64_t n) {
  ra_posmap r{};
  int64_t base = 0;
  for (int i = 0; i < m.nseg; ++i) {
    const ra_seg& g = m.seg[i];
    const int64_t lo = std::max(c0, base), hi = std::min(c0 + n, base + g.len);
    if (lo < hi) r.seg[r.nseg++] = ra_seg{g.begin + (lo - base) * g.stride, g.stride, hi - lo};
    base += g.len;
  }
  if (r.nseg == 0) r = ra_posmap{1, {ra_seg{0, 1, 0}, ra_seg{0, 1, 0}}};
  return r;
}

// dS^T bytes of the stored-dS path in the default workspace: one piece's (in
// chunks when its slices would reach 4 GiB), or every piece's side by side for
// the grouped launches of a per-sequence layout (bf16; fp32 stores none).
static size_t ds_bytes_ring(const std::vector<Piece>& pieces) {
  if (pieces.size() > 1) return ds_bytes_sum(pieces);
  return pieces.empty() ? 0 : ds_default_bytes(&pieces[0].prob, pieces[0].L, pieces[0].L);
}

size_t ra_ring_workspace_bytes(const ra_problem* prob, ra_layout layout, int32_t world) {
  const size_t base = ra_ring_workspace_min_bytes(prob, layout, world);
  if (base == 0) return 0;
  int64_t L = 0;
  std::vector<Piece> pieces;
  ring_common(prob, layout, world, 0, &L, &pieces);
  return base + ds_bytes_ring(pieces);
}

// The ring backward behind ra_ring_bwd and ra_ring_bwd_noalloc.  With
// side_streams false the fp32 per-sequence rings run one after another on the
// caller's stream (no side streams or events are created).
static ra_status ring_bwd_impl(const ra_problem* prob, ra_layout layout, int32_t world, int32_t rank,
                               ra_tensor q_local, ra_tensor k_ring, ra_tensor v_ring, int64_t stride_rank,
                               ra_tensor out, const float* lse, ra_tensor dout, ra_tensor dq, ra_tensor dk_ring,
                               ra_tensor dv_ring, int64_t stride_rank_grad, void* workspace, size_t workspace_bytes,
                               bool side_streams, void* stream) {
  int64_t L = 0;
  std::vector<Piece> pieces;
  ra_status st = ring_common(prob, layout, world, rank, &L, &pieces);
  if (st != RA_OK) return st;
  if (L == 0) return RA_OK;
  const size_t esz = elem_size(prob->dtype);
  if ((st = check_tensor("q_local", q_local, esz, L, true)) != RA_OK) return st;
  if ((st = check_tensor("k_ring", k_ring, esz, L, true)) != RA_OK) return st;
  if ((st = check_tensor("v_ring", v_ring, esz, L, true)) != RA_OK) return st;
  if ((st = check_out_tensor("out", out, 4, true)) != RA_OK) return st;
  if ((st = check_tensor("dout", dout, esz, L, true)) != RA_OK) return st;
  if ((st = check_out_tensor("dq", dq, 4, true)) != RA_OK) return st;
  if ((st = check_out_tensor("dk_ring", dk_ring, 4, true)) != RA_OK) return st;
  if ((st = check_out_tensor("dv_ring", dv_ring, 4, true)) != RA_OK) return st;
  if ((st = check_ptr("lse", lse)) != RA_OK) return st;
  RA_CHECK(stride_rank >= 0 && stride_rank % (int64_t)(16 / esz) == 0, RA_ERR_INVALID_ARG,
           "stride_rank must be >= 0 and keep 16-byte alignment");
  RA_CHECK(stride_rank_grad >= 0 && stride_rank_grad % 4 == 0, RA_ERR_INVALID_ARG,
           "stride_rank_grad must be >= 0 and keep 16-byte alignment");
  const size_t need = ra_ring_workspace_min_bytes(prob, layout, world);
  RA_CHECK(workspace != nullptr && workspace_bytes >= need, RA_ERR_WORKSPACE,
           "workspace of %zu bytes required (got %zu)", need, workspace_bytes);
  RA_CHECK(((uintptr_t)workspace & 15) == 0, RA_ERR_INVALID_ARG, "workspace not 16-byte aligned");
  // The dS^T buffer when the workspace holds it (one piece: in chunks of kc
  // keys when it holds less than the whole block), else none (then dQ comes
  // from the recompute kernel).
  uint16_t* const ds_buf = (uint16_t*)((char*)workspace + need);
  const size_t avail = workspace_bytes - need;
  int64_t kc = 0;
  uint16_t* dsT = nullptr;
  if (pieces.size() == 1) {
    kc = ds_chunk_keys(&pieces[0].prob, pieces[0].L, pieces[0].L, avail);
    dsT = kc > 0 ? ds_buf : nullptr;
  } else {
    const size_t dsb = ds_bytes_sum(pieces);
    dsT = (dsb > 0 && avail >= dsb) ? ds_buf : nullptr;
  }

  float* delta = (float*)workspace;
  hipStream_t s = (hipStream_t)stream;
  const bool bf16 = prob->dtype == RA_DTYPE_BF16;

  PrepArgs pa{};
  pa.out = rd(out);
  pa.dout = rd(dout);
  pa.delta = delta;
  pa.batch = prob->batch;
  pa.heads = prob->heads;
  pa.lq = (int32_t)L;
  pa.dim = prob->head_dim;
  RA_HIP(timed(K_PREP, -1, s, [&] { return launch_prep(pa, bf16, s); }));
  Tensor4W dqw = wr(dq);
  RA_HIP(timed(K_ZERO, -1, s, [&] {
    return launch_zero(dqw, prob->batch, prob->heads, (int32_t)L, prob->head_dim, s);
  }));
  const ra_layout lay = base_layout(layout);
  if (pieces.empty()) return RA_OK;
  if (pieces.size() > 1 && bf16) {
    // Grouped: per ring step one dK/dV launch and one dQ launch over every
    // sequence with visible pairs at that step; each sequence has its own
    // dS^T region, side by side in the workspace.
    const std::vector<PiecePlan> plans = plan_pieces(pieces, lay, world, rank);
    std::vector<int64_t> ds_off(pieces.size(), 0);
    for (size_t i = 1; i < pieces.size(); ++i)
      ds_off[i] = ds_off[i - 1] + (int64_t)(ds_bytes(&pieces[i - 1].prob, pieces[i - 1].L) / 2);
    const ra_problem* p0 = &pieces[0].prob;
    for (int step = 0; step < world; ++step) {
      const int src = ((rank - step) % world + world) % world;
      for (const std::vector<int>& grp : step_groups(pieces, plans, step, true)) {
        BwdArgs a;
        bwd_args(p0, q_local, L, plans[grp[0]].qmap, offset_rd(k_ring, src * stride_rank, esz),
                 offset_rd(v_ring, src * stride_rank, esz), L, plans[grp[0]].kmap[step], dout, lse, delta, wr(dq),
                 offset_wr(dk_ring, src * stride_rank_grad, 4), offset_wr(dv_ring, src * stride_rank_grad, 4), &a);
        a.lse_sh = L;
        a.dsT = dsT;
        a.g.n = (int32_t)grp.size();
        for (size_t j = 0; j < grp.size(); ++j) {
          const int i = grp[j];
          a.g.row0[j] = (int32_t)pieces[i].row0;
          a.g.len[j] = (int32_t)pieces[i].L;
          a.g.qmap[j] = to_dmap(plans[i].qmap);
          a.g.kmap[j] = to_dmap(plans[i].kmap[step]);
          a.g.ds_off[j] = ds_off[i];
          a.g.ds_ld[j] = ds_ld_of(pieces[i].L);
          a.g.qoff[j] = first_seeing_row(pieces[i], plans[i].qmap, plans[i].kmap[step]);  // dQ launch only
        }
        if ((st = launch_bwd_step(a, p0->head_dim, true, step, s)) != RA_OK) return st;
      }
    }
    return RA_OK;
  }
  // one ring: on the caller's stream; fp32 sequences: one ring each on side streams
  // (or one after another on the caller's stream)
  const int ns = (pieces.size() <= 1 || !side_streams) ? 1 : (int)std::min<size_t>(kSideStreams, pieces.size());
  SidePool* pool = nullptr;
  std::vector<int> where(pieces.size(), 0);
  if (ns > 1) {
    if ((st = side_pool(&pool)) != RA_OK) return st;
    where = assign_pieces(pieces, ns);
    if ((st = fork_streams(pool, ns, s)) != RA_OK) return st;
  }
  auto run_piece = [&](const Piece& pc, hipStream_t ps, uint16_t* dsT, int64_t kc) -> ra_status {
    const ra_problem* pp = &pc.prob;
    const ra_tensor qp = shift_rows(q_local, pc.row0, esz), kp = shift_rows(k_ring, pc.row0, esz);
    const ra_tensor vp = shift_rows(v_ring, pc.row0, esz), dop = shift_rows(dout, pc.row0, esz);
    const ra_tensor dqp = shift_rows(dq, pc.row0, 4), dkp = shift_rows(dk_ring, pc.row0, 4);
    const ra_tensor dvp = shift_rows(dv_ring, pc.row0, 4);
    ra_posmap qmap;
    make_posmap(lay, pp->seq_len, world, rank, &qmap);
    for (int step = 0; step < world; ++step) {
      const int src = ((rank - step) % world + world) % world;
      ra_posmap kmap;
      make_posmap(lay, pp->seq_len, world, src, &kmap);
      if (!step_has_pairs(pp, qmap, pc.L, kmap, pc.L)) continue;
      // the step's keys in chunks of kc (one chunk without a dS^T buffer)
      const int64_t ck = (dsT && kc > 0) ? kc : pc.L;
      for (int64_t c0 = 0; c0 < pc.L; c0 += ck) {
        const int64_t n = std::min(ck, pc.L - c0);
        const ra_posmap km = n == pc.L ? kmap : sub_posmap(kmap, c0, n);
        if (!step_has_pairs(pp, qmap, pc.L, km, n)) continue;
        BwdArgs a;
        bwd_args(pp, qp, pc.L, qmap, offset_rd(shift_rows(kp, c0, esz), src * stride_rank, esz),
                 offset_rd(shift_rows(vp, c0, esz), src * stride_rank, esz), n, km, dop, lse + pc.row0,
                 delta + pc.row0, wr(dqp), offset_wr(shift_rows(dkp, c0, 4), src * stride_rank_grad, 4),
                 offset_wr(shift_rows(dvp, c0, 4), src * stride_rank_grad, 4), &a);
        a.lse_sh = L;
        a.dsT = dsT;
        a.ds_ld = ds_ld_of(pc.L);
        ra_status st2 = launch_bwd_step(a, pp->head_dim, bf16, step, ps);
        if (st2 != RA_OK) return st2;
      }
    }
    return RA_OK;
  };
  if (pieces.size() == 1) return run_piece(pieces[0], s, dsT, kc);
  if (ns == 1) {
    for (size_t i = 0; i < pieces.size() && st == RA_OK; ++i) st = run_piece(pieces[i], s, nullptr, 0);
    return st;
  }
  for (size_t i = 0; i < pieces.size() && st == RA_OK; ++i)
    st = run_piece(pieces[i], pool->st[where[i]], nullptr, 0);
  const ra_status sj = join_streams(pool, ns, s);
  return st != RA_OK ? st : sj;
}

ra_status ra_ring_bwd(const ra_problem* prob, ra_layout layout, int32_t world, int32_t rank, ra_tensor q_local,
                      ra_tensor k_ring, ra_tensor v_ring, int64_t stride_rank, ra_tensor out, const float* lse,
                      ra_tensor dout, ra_tensor dq, ra_tensor dk_ring, ra_tensor dv_ring, int64_t stride_rank_grad,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return ring_bwd_impl(prob, layout, world, rank, q_local, k_ring, v_ring, stride_rank, out, lse, dout, dq, dk_ring,
                       dv_ring, stride_rank_grad, workspace, workspace_bytes, true, stream);
}

size_t ra_noalloc_scratch_bytes(void) { return scratch_capacity(); }

ra_status ra_ring_bwd_noalloc(const ra_problem* prob, ra_layout layout, int32_t world, int32_t rank,
                              ra_tensor q_local, ra_tensor k_ring, ra_tensor v_ring, int64_t stride_rank,
                              ra_tensor out, const float* lse, ra_tensor dout, ra_tensor dq, ra_tensor dk_ring,
                              ra_tensor dv_ring, int64_t stride_rank_grad, void* stream) {
  // Validation and the size check first (host arithmetic only): delta must fit
  // the fixed scratch.
  int64_t L = 0;
  std::vector<Piece> pieces;
  ra_status st = ring_common(prob, layout, world, rank, &L, &pieces);
  if (st != RA_OK) return st;
  if (L == 0) return RA_OK;
  const size_t cap = scratch_capacity();
  const size_t need = ra_ring_workspace_min_bytes(prob, layout, world);
  RA_CHECK(need <= cap, RA_ERR_WORKSPACE,
           "ra_ring_bwd_noalloc: delta needs %zu bytes, more than the %zu-byte fixed scratch "
           "(batch*heads*S/N must stay at or below %zu); use ra_ring_bwd with a workspace",
           need, cap, cap / sizeof(float));
  void* ptr = nullptr;
  RA_HIP(scratch_device_ptr(&ptr));
  return ring_bwd_impl(prob, layout, world, rank, q_local, k_ring, v_ring, stride_rank, out, lse, dout, dq, dk_ring,
                       dv_ring, stride_rank_grad, ptr, cap, false, stream);
}


// ---- gathered K/V share (llama3-style context parallelism) --------------------------------
//
// Every rank holds the whole K/V in global token order (all-gathered) and
// attends its local queries to it as ONE block step (SourcePulse page on
// ring-flash-attention, "How It Works" and "Highlighted Details").  Only the
// key range the rank's queries can see is handed to the kernels: under the
// causal mask nothing past the last query position, and with cu_seqlens
// nothing before the start of the first query's sequence (or past the end of
// the last one's).

static ra_status gathered_common(const ra_problem* prob, ra_layout layout, int32_t world, int32_t rank,
                                 ra_posmap* qmap, int64_t* L, int64_t* k_lo, int64_t* nk) {
  ra_status st = check_problem(prob);
  if (st != RA_OK) return st;
  RA_CHECK(layout == RA_LAYOUT_CONTIGUOUS || layout == RA_LAYOUT_ZIGZAG || layout == RA_LAYOUT_STRIPE,
           RA_ERR_UNSUPPORTED, "gathered share: layout %d not supported (contiguous, zigzag or stripe)",
           (int)layout);
  if ((st = make_posmap(layout, prob->seq_len, world, rank, qmap)) != RA_OK) return st;
  *L = prob->seq_len / world;
  *k_lo = 0;
  *nk = 0;
  if (*L == 0) return RA_OK;
  const int64_t qmin = pos_at(*qmap, 0), qmax = pos_at(*qmap, *L - 1);
  int64_t lo = 0, hi = prob->causal ? qmax : prob->seq_len - 1;
  if (prob->num_seqs > 0 && prob->cu_seqlens_host) {
    const int32_t* cu = prob->cu_seqlens_host;
    const int32_t* f = std::upper_bound(cu, cu + prob->num_seqs + 1, (int32_t)qmin);
    lo = f[-1];  // start of the first query's sequence
    if (!prob->causal) {
      const int32_t* g = std::upper_bound(cu, cu + prob->num_seqs + 1, (int32_t)qmax);
      hi = (g <= cu + prob->num_seqs ? *g : prob->seq_len) - 1;  // end of the last query's sequence
    }
  }
  *k_lo = lo;
  *nk = hi - lo + 1;
  return RA_OK;
}

// dS^T bytes of a gathered share: b*h slices of round_up(nk, 128) keys x round_up(L, 128)
// rows (bf16), 0 when not applicable (fp32, or a slice beyond 32-bit byte offsets).
static size_t gathered_ds_bytes(const ra_problem* prob, int64_t L, int64_t nk) {
  return nk > 0 ? ds_default_bytes(prob, L, nk) : 0;
}

size_t ra_gathered_workspace_min_bytes(const ra_problem* prob, ra_layout layout, int32_t world, int32_t rank) {
  ra_posmap qm;
  int64_t L = 0, k_lo = 0, nk = 0;
  if (gathered_common(prob, layout, world, rank, &qm, &L, &k_lo, &nk) != RA_OK) return 0;
  const size_t bytes = (size_t)prob->batch * prob->heads * L * sizeof(float);
  return (bytes + 255) & ~(size_t)255;
}

size_t ra_gathered_workspace_bytes(const ra_problem* prob, ra_layout layout, int32_t world, int32_t rank) {
  ra_posmap qm;
  int64_t L = 0, k_lo = 0, nk = 0;
  if (gathered_common(prob, layout, world, rank, &qm, &L, &k_lo, &nk) != RA_OK) return 0;
  const size_t base = ((size_t)prob->batch * prob->heads * L * sizeof(float) + 255) & ~(size_t)255;
  return base + gathered_ds_bytes(prob, L, nk);
}

ra_status ra_gathered_fwd(const ra_problem* prob, ra_layout layout, int32_t world, int32_t rank, ra_tensor q_local,
                          ra_tensor k_all, ra_tensor v_all, ra_tensor out, float* lse, ra_tensor out_lowp,
                          void* stream) {
  ra_posmap qmap;
  int64_t L = 0, k_lo = 0, nk = 0;
  ra_status st = gathered_common(prob, layout, world, rank, &qmap, &L, &k_lo, &nk);
  if (st != RA_OK) return st;
  if (L == 0) return RA_OK;
  const size_t esz = elem_size(prob->dtype);
  if ((st = check_tensor("q_local", q_local, esz, L, true)) != RA_OK) return st;
  if ((st = check_tensor("k_all", shift_rows(k_all, k_lo, esz), esz, nk, true)) != RA_OK) return st;
  if ((st = check_tensor("v_all", shift_rows(v_all, k_lo, esz), esz, nk, true)) != RA_OK) return st;
  if ((st = check_out_tensor("out", out, 4, true)) != RA_OK) return st;
  if ((st = check_out_tensor("out_lowp", out_lowp, esz, out_lowp.ptr != nullptr)) != RA_OK) return st;
  if ((st = check_ptr("lse", lse)) != RA_OK) return st;
  const ra_posmap kmap{1, {ra_seg{k_lo, 1, nk}, ra_seg{0, 1, 0}}};
  FwdArgs a{};
  a.q = rd(q_local);
  a.k = rd(shift_rows(k_all, k_lo, esz));
  a.v = rd(shift_rows(v_all, k_lo, esz));
  a.out = wr(out);
  a.lse = lse;
  a.lse_sh = L;
  a.out_lowp = wr(out_lowp);
  a.batch = prob->batch;
  a.heads = prob->heads;
  a.lq = (int32_t)L;
  a.lk = (int32_t)nk;
  a.qmap = to_dmap(qmap);
  a.kmap = to_dmap(kmap);
  a.mask = mask_of(prob);
  a.scale_log2 = scale_of(prob) * 1.4426950408889634f;
  a.mode = FWD_STORE;
  a.n_qtiles = ceil_div(L, FWD_BQ);
  hipStream_t s = (hipStream_t)stream;
  const bool bf16 = prob->dtype == RA_DTYPE_BF16;
  RA_HIP(timed(K_FWD, 0, s, [&] { return launch_fwd(a, prob->head_dim, bf16, s); }));
  return RA_OK;
}

ra_status ra_gathered_bwd(const ra_problem* prob, ra_layout layout, int32_t world, int32_t rank, ra_tensor q_local,
                          ra_tensor k_all, ra_tensor v_all, ra_tensor out, const float* lse, ra_tensor dout,
                          ra_tensor dq, ra_tensor dk_all, ra_tensor dv_all, void* workspace, size_t workspace_bytes,
                          void* stream) {
  ra_posmap qmap;
  int64_t L = 0, k_lo = 0, nk = 0;
  ra_status st = gathered_common(prob, layout, world, rank, &qmap, &L, &k_lo, &nk);
  if (st != RA_OK) return st;
  if (L == 0) return RA_OK;
  const size_t esz = elem_size(prob->dtype);
  if ((st = check_tensor("q_local", q_local, esz, L, true)) != RA_OK) return st;
  if ((st = check_tensor("k_all", shift_rows(k_all, k_lo, esz), esz, nk, true)) != RA_OK) return st;
  if ((st = check_tensor("v_all", shift_rows(v_all, k_lo, esz), esz, nk, true)) != RA_OK) return st;
  if ((st = check_out_tensor("out", out, 4, true)) != RA_OK) return st;
  if ((st = check_tensor("dout", dout, esz, L, true)) != RA_OK) return st;
  if ((st = check_out_tensor("dq", dq, 4, true)) != RA_OK) return st;
  if ((st = check_out_tensor("dk_all", shift_rows(dk_all, k_lo, 4), 4, true)) != RA_OK) return st;
  if ((st = check_out_tensor("dv_all", shift_rows(dv_all, k_lo, 4), 4, true)) != RA_OK) return st;
  if ((st = check_ptr("lse", lse)) != RA_OK) return st;
  const size_t need = ra_gathered_workspace_min_bytes(prob, layout, world, rank);
  RA_CHECK(workspace != nullptr && workspace_bytes >= need, RA_ERR_WORKSPACE,
           "workspace of %zu bytes required (got %zu)", need, workspace_bytes);
  RA_CHECK(((uintptr_t)workspace & 15) == 0, RA_ERR_INVALID_ARG, "workspace not 16-byte aligned");
  // dS^T in chunks of kc keys when the workspace holds less than the whole block
  const int64_t kc = ds_chunk_keys(prob, L, nk, workspace_bytes - need);
  uint16_t* dsT = kc > 0 ? (uint16_t*)((char*)workspace + need) : nullptr;
  float* delta = (float*)workspace;
  hipStream_t s = (hipStream_t)stream;
  const bool bf16 = prob->dtype == RA_DTYPE_BF16;

  PrepArgs pa{};
  pa.out = rd(out);
  pa.dout = rd(dout);
  pa.delta = delta;
  pa.batch = prob->batch;
  pa.heads = prob->heads;
  pa.lq = (int32_t)L;
  pa.dim = prob->head_dim;
  RA_HIP(timed(K_PREP, -1, s, [&] { return launch_prep(pa, bf16, s); }));
  Tensor4W dqw = wr(dq);
  RA_HIP(timed(K_ZERO, -1, s, [&] {
    return launch_zero(dqw, prob->batch, prob->heads, (int32_t)L, prob->head_dim, s);
  }));
  // the visible keys [k_lo, k_lo + nk) in chunks of kc (one chunk without a dS^T buffer)
  const int64_t ck = dsT ? kc : nk;
  for (int64_t c0 = 0; c0 < nk; c0 += ck) {
    const int64_t n = std::min(ck, nk - c0), k0 = k_lo + c0;
    const ra_posmap kmap{1, {ra_seg{k0, 1, n}, ra_seg{0, 1, 0}}};
    if (n < nk && !step_has_pairs(prob, qmap, L, kmap, n)) continue;
    BwdArgs a;
    bwd_args(prob, q_local, L, qmap, rd(shift_rows(k_all, k0, esz)), rd(shift_rows(v_all, k0, esz)), n, kmap, dout,
             lse, delta, dqw, wr(shift_rows(dk_all, k0, 4)), wr(shift_rows(dv_all, k0, 4)), &a);
    a.dsT = dsT;
    a.ds_ld = ds_ld_of(L);
    if ((st = launch_bwd_step(a, prob->head_dim, bf16, 0, s)) != RA_OK) return st;
  }
  return RA_OK;
}

}  // extern "C"
