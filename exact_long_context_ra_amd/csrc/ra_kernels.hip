// gfx950 (MI355X) kernels for the ring-attention per-device hot path.
//
// Forward block step ("Ring Flash Attention" README: each block returns its
// output and softmax_lse; guijiagi.com Ring Attention article, online-softmax
// section: running max / running sum rescaling) and its backward (textbook
// softmax-attention gradient with P recomputed from the final lse).
//
// MFMA orientation.  A forward wave computes S^T = K * Q^T (M = 32 keys, N =
// 32 queries) so that in the MFMA result layout every lane holds ONE query
// and 16 keys: the row max / row sum of the online softmax are per-lane
// reductions plus one exchange between the two 32-lane halves.  The A-operand
// rows (keys) are permuted (bits 2 and 3 of the row index swapped) so that the
// result registers of each half are 8 consecutive keys, which is exactly the
// B-operand layout of the next product O^T += V^T * P^T (K-dim = keys).
//
// Two families of kernels:
//  * bf16 inputs (the measured path): fwd_kernel_bf16 (4 waves, 128 query
//    rows, 64-key tiles), bwd_dkdv_kernel (8 waves, 128 keys, 64-row query
//    tiles; stores dS), bwd_dq_ds_kernel (dQ = dS K from the stored dS) and
//    bwd_dq_kernel (dQ with S and dP recomputed, when there is no room for
//    dS).  Tiles are copied by buffer->LDS DMA in natural [row][d] layout with
//    XOR-swizzled 16-byte chunks; transposed operands come from
//    ds_read_b64_tr_b16.
//  * fp32 inputs (the tight-tolerance parity path): fwd_kernel<D, false> and
//    the fused bwd_kernel<D, false>, with register-staged tiles (V stored
//    transposed in LDS), fp32 MFMA, and dQ added with fp32 atomics.
//
// Masks are evaluated on global token positions (see ra.h): per query row a
// visible key interval [lo, hi] follows from the causal flag and cu_seqlens;
// tiles entirely outside it are skipped, tiles entirely inside it run without
// any per-element mask, and only the remaining tiles are masked per element.
#include <mutex>
#include <type_traits>

#include "ra_internal.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int NT = 256;  // threads per workgroup (4 waves of 64)
constexpr float NEG_INF = -__builtin_huge_valf();
constexpr float POS_INF = __builtin_huge_valf();
constexpr float LN2 = 0.69314718055994531f;
constexpr float LOG2E = 1.4426950408889634f;
constexpr int INT_BIG = 0x7fffffff;

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 ld_bf16x8(const void* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ bf16x8 zero_bf16x8() { return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u}); }

// A-operand row permutation: swap bits 2 and 3 of the row index.
__device__ __forceinline__ int row_perm(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }
// Physical row (within a 32-row block) held by result register v of half hf
// when the A rows were permuted by row_perm.
__device__ __forceinline__ int reg_row(int v, int hf) { return (v < 8) ? (8 * hf + v) : (16 + 8 * hf + (v - 8)); }

// Byte offset in a transposed tile with 64 entries (128 bytes) per row: the
// 16-byte chunk index is XOR-swizzled by the row so that both the 16-byte
// MFMA-operand reads (32 rows, same chunk) and the 8-byte transposing writes
// stay (nearly) bank-conflict free.
__device__ __forceinline__ int tr_off(int row, int col) {
  int sw = ((row >> 1) ^ (row >> 3)) & 7;
  return row * 128 + ((((col >> 3) ^ sw)) << 4) + ((col & 7) << 1);
}

// Value of lane l ^ 32 combined with lane l's own, for both halves of the
// wave at once: v_permlane32_swap exchanges the upper 32 lanes of one register
// with the lower 32 of another, so swapping a copy with itself gives every lane
// the pair (x[l], x[l ^ 32]) in its two results, in VALU time (a cross-lane
// read through the LDS crossbar would sit on the path from the scores to the
// exponentials).
__device__ __forceinline__ float max_halves(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// ---- posmaps and visibility ---------------------------------------------------------------

__device__ __forceinline__ int map_pos(const DMap& m, int a) {
  return (a < m.s0.len) ? m.s0.begin + a * m.s0.stride : m.s1.begin + (a - m.s0.len) * m.s1.stride;
}
// Unit-stride segments (contiguous and zigzag chunks) need no division.
__device__ __forceinline__ int seg_first_ge(const DSeg& s, int P) {
  if (s.len <= 0) return 0;
  if (P <= s.begin) return 0;
  if (s.stride == 1) return min(P - s.begin, s.len);
  long long last = (long long)s.begin + (long long)(s.len - 1) * s.stride;
  if (last < P) return s.len;
  return (int)(((long long)P - s.begin + s.stride - 1) / s.stride);
}
__device__ __forceinline__ int seg_last_le(const DSeg& s, int P) {
  if (s.len <= 0 || P < s.begin) return -1;
  if (s.stride == 1) return min(P - s.begin, s.len - 1);
  long long i = ((long long)P - s.begin) / s.stride;
  return (int)(i < s.len - 1 ? i : s.len - 1);
}
// First local index whose position is >= P (total if none).
__device__ __forceinline__ int first_ge(const DMap& m, int P) {
  int i = seg_first_ge(m.s0, P);
  if (i < m.s0.len || m.nseg < 2) return i;
  return m.s0.len + seg_first_ge(m.s1, P);
}
// Last local index whose position is <= P (-1 if none).
__device__ __forceinline__ int last_le(const DMap& m, int P) {
  if (m.nseg == 2) {
    int i = seg_last_le(m.s1, P);
    if (i >= 0) return m.s0.len + i;
  }
  return seg_last_le(m.s0, P);
}

// Largest k in [0, nseq) with cu[k] <= p.
__device__ __forceinline__ int seq_index(const MaskSpec& ms, int p) {
  int lo = 0, hi = ms.nseq - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (ms.cu[mid] <= p) lo = mid; else hi = mid - 1;
  }
  return lo;
}

struct Bounds { int lo, hi; };

// Visible key positions for a query at global position qp.
__device__ __forceinline__ Bounds row_bounds(const MaskSpec& ms, int qp) {
  Bounds b;
  if (ms.nseq > 0) {
    int k = seq_index(ms, qp);
    b.lo = ms.cu[k];
    b.hi = ms.causal ? qp : ms.cu[k + 1] - 1;
  } else {
    b.lo = 0;
    b.hi = ms.causal ? qp : INT_BIG;
  }
  return b;
}
// Query positions that can see a key at global position kp.
__device__ __forceinline__ Bounds col_bounds(const MaskSpec& ms, int kp) {
  Bounds b;
  if (ms.nseq > 0) {
    int k = seq_index(ms, kp);
    b.lo = ms.causal ? kp : ms.cu[k];
    b.hi = ms.cu[k + 1] - 1;
  } else {
    b.lo = ms.causal ? kp : 0;
    b.hi = INT_BIG;
  }
  return b;
}

// Workgroup id -> logical id, so that consecutive logical ids (same head) land
// on the same XCD (ids are dispatched round-robin over the 8 XCDs) and share
// that XCD's L2 for the head's K/V.
__device__ __forceinline__ int xcd_logical(int bid, int total) {
  if ((total & 7) != 0) return bid;
  return (bid & 7) * (total >> 3) + (bid >> 3);
}

// The posmap of local indices [n0, total) of m (0 <= n0 < total).
__device__ __forceinline__ DMap dmap_tail(const DMap& m, int n0) {
  DMap r = m;
  if (n0 <= 0) return r;
  if (n0 < m.s0.len) {
    r.s0.begin += n0 * m.s0.stride;
    r.s0.len -= n0;
  } else {
    const int k = n0 - m.s0.len;
    r.nseg = 1;
    r.s0 = DSeg{m.s1.begin + k * m.s1.stride, m.s1.stride, m.s1.len - k};
    r.s1 = DSeg{0, 1, 0};
  }
  r.total = m.total - n0;
  return r;
}

// Block of a grouped launch (a table of independent rings, see PieceTable):
// finds this block's piece, points the row-based tensors at its rows and sets
// its lengths, posmaps and flags; bid/nblk become the block index and count
// within the piece.  bf16 operands, fp32 outputs and accumulators.
__device__ __forceinline__ int piece_of(const PieceTable& g, int x) {
  int p = 0;
  while (p + 1 < g.n && g.wg_begin[p + 1] <= x) ++p;
  return p;
}
__device__ __forceinline__ void fwd_piece(const FwdArgs& ap, FwdArgs& a, int& bid, int& nblk) {
  const PieceTable& g = ap.g;
  const int p = piece_of(g, (int)blockIdx.x);
  bid = (int)blockIdx.x - g.wg_begin[p];
  nblk = g.wg_begin[p + 1] - g.wg_begin[p];
  const int64_t r0 = g.row0[p];
  const int qo = g.qoff[p];
  const int64_t q0 = r0 + qo;  // first query row of this launch
  const int f = g.flags[p];
  a.q.ptr = reinterpret_cast<const char*>(ap.q.ptr) + q0 * ap.q.st * 2;
  a.k.ptr = reinterpret_cast<const char*>(ap.k.ptr) + r0 * ap.k.st * 2;
  a.v.ptr = reinterpret_cast<const char*>(ap.v.ptr) + r0 * ap.v.st * 2;
  a.out.ptr = reinterpret_cast<char*>(ap.out.ptr) + q0 * ap.out.st * 4;
  a.out_lowp.ptr = (f & PIECE_LOWP) ? reinterpret_cast<char*>(ap.out_lowp.ptr) + q0 * ap.out_lowp.st * 2 : nullptr;
  a.lse = ap.lse + q0;
  a.lq = g.len[p] - qo;
  a.lk = g.len[p];
  a.qmap = dmap_tail(g.qmap[p], qo);
  a.kmap = g.kmap[p];
  a.mode = (f & PIECE_MERGE) ? FWD_MERGE : FWD_STORE;
  a.n_qtiles = (a.lq + FWD_BQ - 1) / FWD_BQ;
}
// `qside`: the dQ kernels take the piece's query rows from qoff on; the dK/dV
// kernel takes them all.
__device__ __forceinline__ void bwd_piece(const BwdArgs& ap, BwdArgs& a, int& bid, int& nblk, bool qside) {
  const PieceTable& g = ap.g;
  const int p = piece_of(g, (int)blockIdx.x);
  bid = (int)blockIdx.x - g.wg_begin[p];
  nblk = g.wg_begin[p + 1] - g.wg_begin[p];
  const int64_t r0 = g.row0[p];
  const int qo = qside ? g.qoff[p] : 0;
  const int64_t q0 = r0 + qo;  // first query row of this launch
  a.q.ptr = reinterpret_cast<const char*>(ap.q.ptr) + q0 * ap.q.st * 2;
  a.k.ptr = reinterpret_cast<const char*>(ap.k.ptr) + r0 * ap.k.st * 2;
  a.v.ptr = reinterpret_cast<const char*>(ap.v.ptr) + r0 * ap.v.st * 2;
  a.dout.ptr = reinterpret_cast<const char*>(ap.dout.ptr) + q0 * ap.dout.st * 2;
  a.dq.ptr = reinterpret_cast<char*>(ap.dq.ptr) + q0 * ap.dq.st * 4;
  a.dk.ptr = reinterpret_cast<char*>(ap.dk.ptr) + r0 * ap.dk.st * 4;
  a.dv.ptr = reinterpret_cast<char*>(ap.dv.ptr) + r0 * ap.dv.st * 4;
  a.lse = ap.lse + q0;
  a.delta = ap.delta + q0;
  a.lq = g.len[p] - qo;
  a.lk = g.len[p];
  a.qmap = dmap_tail(g.qmap[p], qo);
  a.kmap = g.kmap[p];
  a.n_ktiles = (a.lk + BWD_BK - 1) / BWD_BK;
  a.n_qtiles = (a.lq + FWD_BQ - 1) / FWD_BQ;
  a.dsT = ap.dsT ? ap.dsT + g.ds_off[p] : nullptr;
  a.ds_ld = g.ds_ld[p];
  a.ds_row0 = qo;
}

// ============================================================================================
// Buffer loads.  Each (batch, head) slice of a tensor gets a range-checked
// buffer descriptor; a read past the slice returns zeros, so ragged tiles need
// neither branches nor clamped addresses (and the loads of a tile can all be
// in flight at once).
// ============================================================================================

typedef __amdgpu_buffer_rsrc_t Rsrc;

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(Rsrc r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ f32x4 bload16f(Rsrc r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ float bload4f(Rsrc r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ uint16_t bload2(Rsrc r, uint32_t off) {
  return __builtin_bit_cast(uint16_t, __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
}
// Bytes spanned by `rows` rows of `dim` elements at a stride of `st` elements.
__device__ __forceinline__ uint32_t slice_bytes(int rows, int64_t st, int esz, int dim) {
  return rows <= 0 ? 0u : (uint32_t)((int64_t)(rows - 1) * st * esz + (int64_t)dim * esz);
}

// ============================================================================================
// Forward
// ============================================================================================

constexpr int FBK = 64;             // keys per forward tile
constexpr float RESCALE_TH = 8.f;   // rescale O only when a row max grows by more than 2^8

template <int D, bool BF16>
struct FwdCfg {
  // bf16: K rows padded by 16 bytes; V^T rows of 64 keys, swizzled; two buffers.
  // fp32: K rows padded by 2 floats, V rows padded by 4 floats; one buffer.
  static constexpr int KSTR = BF16 ? (D + 8) * 2 : (D + 2) * 4;
  static constexpr int VSZ = BF16 ? D * 128 : FBK * (D + 4) * 4;
  static constexpr int VSTR = (D + 4) * 4;  // fp32 V row stride
  static constexpr int BUF = FBK * KSTR + VSZ;
  static constexpr int NBUF = BF16 ? 2 : 1;
  static constexpr int LDS = NBUF * BUF;
};

// bf16 K/V tile: global -> registers (issued one tile ahead) -> LDS.
template <int D>
struct KVStageBf16 {
  static constexpr int CPR = D / 8;     // 16-byte chunks per row
  static constexpr int RPP = NT / CPR;  // K rows per pass
  static constexpr int KP = FBK / RPP;  // K passes
  static constexpr int VITEMS = (FBK / 4) * CPR;  // (4 keys x 8 d) items of V
  u32x4 k[KP];
  u32x4 v[4];

  __device__ __forceinline__ void load(Rsrc rk, Rsrc rv, uint32_t kst, uint32_t vst, int j0, int tid) {
#pragma unroll
    for (int p = 0; p < KP; ++p) {
      const int r = p * RPP + tid / CPR, c = tid % CPR;
      k[p] = bload16(rk, (uint32_t)(j0 + r) * kst + c * 16);
    }
    if (tid < VITEMS) {
      const int c = tid % CPR, kq = tid / CPR;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = bload16(rv, (uint32_t)(j0 + 4 * kq + i) * vst + c * 16);
    }
  }
  __device__ __forceinline__ void store(char* sK, char* sV, int tid) const {
    constexpr int KSTR = FwdCfg<D, true>::KSTR;
#pragma unroll
    for (int p = 0; p < KP; ++p) {
      const int r = p * RPP + tid / CPR, c = tid % CPR;
      *reinterpret_cast<u32x4*>(sK + r * KSTR + c * 16) = k[p];
    }
    if (tid < VITEMS) {
      const int c = tid % CPR, kq = tid / CPR;
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const int e = dd >> 1;
        uint32_t w0, w1;
        if (dd & 1) {
          w0 = (v[0][e] >> 16) | (v[1][e] & 0xffff0000u);
          w1 = (v[2][e] >> 16) | (v[3][e] & 0xffff0000u);
        } else {
          w0 = (v[0][e] & 0xffffu) | (v[1][e] << 16);
          w1 = (v[2][e] & 0xffffu) | (v[3][e] << 16);
        }
        *reinterpret_cast<u32x2*>(sV + tr_off(8 * c + dd, 4 * kq)) = u32x2{w0, w1};
      }
    }
  }
};

template <int D>
__device__ __forceinline__ void fwd_stage_f32(Rsrc rk, Rsrc rv, uint32_t kst, uint32_t vst, int j0, char* sK,
                                              char* sV, int tid) {
  using C = FwdCfg<D, false>;
  constexpr int CPR = D / 4;  // float4 chunks per row
  constexpr int ITEMS = FBK * CPR;
#pragma unroll 4
  for (int it = tid; it < ITEMS; it += NT) {
    const int r = it / CPR, c = it % CPR;
    const f32x4 kv = bload16f(rk, (uint32_t)(j0 + r) * kst + c * 16);
    const f32x4 vv = bload16f(rv, (uint32_t)(j0 + r) * vst + c * 16);
    float* kd = reinterpret_cast<float*>(sK + r * C::KSTR) + c * 4;
    *reinterpret_cast<float2*>(kd) = make_float2(kv[0], kv[1]);
    *reinterpret_cast<float2*>(kd + 2) = make_float2(kv[2], kv[3]);
    *reinterpret_cast<f32x4*>(sV + r * C::VSTR + c * 16) = vv;
  }
}

// One 64-key tile for one wave (32 query rows): S^T, mask, online softmax, O^T += V^T P^T.
template <int D, bool BF16, typename QF>
__device__ __forceinline__ void fwd_tile(const FwdArgs& a, int j0, const char* sK, const char* sV, const QF* qf,
                                         const Bounds& rb, const Bounds& wv_f, const Bounds& wv_l,
                                         bool wave_has_rows, float& m_run, float& l_run, f32x16* o, int l32,
                                         int hf) {
  using C = FwdCfg<D, BF16>;
  constexpr int NDB = D / 32;
  const int jl = min(a.lk, j0 + FBK) - 1;
  const int kmin = map_pos(a.kmap, j0), kmax = map_pos(a.kmap, jl);
  if (!wave_has_rows || kmax < wv_f.lo || kmin > wv_l.hi) return;  // nothing visible to this wave
  const bool wave_full = (j0 + FBK <= a.lk) && kmin >= wv_l.lo && kmax <= wv_f.hi;
  const float sl2 = a.scale_log2;

  f32x16 st[2];
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2) {
    f32x16 acc = f32x16{};
    if constexpr (BF16) {
      const char* kr = sK + (c2 * 32 + row_perm(l32)) * C::KSTR + hf * 16;
#pragma unroll
      for (int c = 0; c < D / 16; ++c) acc = mfma_bf16(ld_bf16x8(kr + c * 32), qf[c], acc);
    } else {
      const float* kr = reinterpret_cast<const float*>(sK + (c2 * 32 + row_perm(l32)) * C::KSTR) + hf;
#pragma unroll
      for (int t = 0; t < D / 2; ++t) acc = mfma_f32(kr[2 * t], qf[t], acc);
    }
    st[c2] = acc;
  }
  if (!wave_full) {
    const bool in0 = j0 < a.kmap.s0.len;
    const bool one_seg = a.kmap.nseg < 2 || in0 == (jl < a.kmap.s0.len);
    const int kstr = in0 ? a.kmap.s0.stride : a.kmap.s1.stride;
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int j = j0 + c2 * 32 + reg_row(v, hf);
        const int kp = one_seg ? kmin + (j - j0) * kstr : map_pos(a.kmap, min(j, jl));
        const bool ok = (j <= jl) && kp >= rb.lo && kp <= rb.hi;
        st[c2][v] = ok ? st[c2][v] : NEG_INF;
      }
  }
  float mx = NEG_INF;
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, st[c2][v]);
  mx = max_halves(mx) * sl2;
  // Lazy rescale: the running max only moves when a row max exceeds it by
  // more than RESCALE_TH (so P <= 2^RESCALE_TH); the result is exact either way.
  const bool grow = mx > m_run + RESCALE_TH;
  if (__any(grow)) {
    const float m_new = grow ? mx : m_run;
    const float alpha = (m_new == m_run) ? 1.f : ex2(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int d = 0; d < NDB; ++d) o[d] *= alpha;
    m_run = m_new;
  }
  const float m_use = (m_run == NEG_INF) ? 0.f : m_run;
  float rs = 0.f;
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float p = ex2(__builtin_fmaf(st[c2][v], sl2, -m_use));
      st[c2][v] = p;
      rs += p;
    }
  l_run += rs;

  // O^T += V^T P^T
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2) {
    if constexpr (BF16) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        bf16x8 pb;
#pragma unroll
        for (int i = 0; i < 8; ++i) pb[i] = (__bf16)st[c2][8 * u + i];
        const int kcol = c2 * 32 + 16 * u + 8 * hf;
#pragma unroll
        for (int d = 0; d < NDB; ++d) o[d] = mfma_bf16(ld_bf16x8(sV + tr_off(d * 32 + l32, kcol)), pb, o[d]);
      }
    } else {
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const float* vr = reinterpret_cast<const float*>(sV + (c2 * 32 + reg_row(t, hf)) * C::VSTR) + l32;
#pragma unroll
        for (int d = 0; d < NDB; ++d) o[d] = mfma_f32(vr[d * 32], st[c2][t], o[d]);
      }
    }
  }
}

template <int D, bool BF16>
__global__ __launch_bounds__(NT, 2) void fwd_kernel(FwdArgs a) {
  using C = FwdCfg<D, BF16>;
  constexpr int NDB = D / 32;
  constexpr int ESZ = BF16 ? 2 : 4;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int logical = xcd_logical(blockIdx.x, gridDim.x);
  const int qt = a.n_qtiles - 1 - logical % a.n_qtiles;  // latest (heaviest causal) tiles first
  const int bh = logical / a.n_qtiles;
  const int head = bh % a.heads, b = bh / a.heads;

  const int r_first = qt * FWD_BQ;
  const int r_last = min(a.lq, r_first + FWD_BQ) - 1;
  const int w_first = r_first + 32 * w;
  const int w_last = min(r_last, w_first + 31);
  const bool wave_has_rows = w_first <= r_last;
  const int row = w_first + l32;
  const bool row_ok = row <= r_last;

  const char* qbase = reinterpret_cast<const char*>(a.q.ptr) + (b * a.q.sb + head * a.q.sh) * ESZ;
  const char* kbase = reinterpret_cast<const char*>(a.k.ptr) + (b * a.k.sb + head * a.k.sh) * ESZ;
  const char* vbase = reinterpret_cast<const char*>(a.v.ptr) + (b * a.v.sb + head * a.v.sh) * ESZ;
  const Rsrc rq = make_rsrc(qbase, slice_bytes(a.lq, a.q.st, ESZ, D));
  const Rsrc rk = make_rsrc(kbase, slice_bytes(a.lk, a.k.st, ESZ, D));
  const Rsrc rv = make_rsrc(vbase, slice_bytes(a.lk, a.v.st, ESZ, D));
  const uint32_t qst = (uint32_t)(a.q.st * ESZ), kst = (uint32_t)(a.k.st * ESZ), vst = (uint32_t)(a.v.st * ESZ);

  // Query fragments (B operand of S^T = K Q^T), kept in registers.
  constexpr int NQF = BF16 ? D / 16 : D / 2;
  typedef typename std::conditional<BF16, bf16x8, float>::type QF;
  QF qf[NQF];
  if constexpr (BF16) {
#pragma unroll
    for (int c = 0; c < NQF; ++c)
      qf[c] = __builtin_bit_cast(bf16x8, bload16(rq, (uint32_t)row * qst + (16 * c + 8 * hf) * 2));
  } else {
#pragma unroll
    for (int c4 = 0; c4 < D / 4; ++c4) {
      const f32x4 x = bload16f(rq, (uint32_t)row * qst + 16 * c4);
      qf[2 * c4] = hf ? x[1] : x[0];
      qf[2 * c4 + 1] = hf ? x[3] : x[2];
    }
  }

  // Visibility bounds: this lane's row, the workgroup's and the wave's extremes.
  const Bounds rb = row_bounds(a.mask, map_pos(a.qmap, min(row, r_last)));
  const Bounds wg_f = row_bounds(a.mask, map_pos(a.qmap, r_first));
  const Bounds wg_l = row_bounds(a.mask, map_pos(a.qmap, r_last));
  const Bounds wv_f = row_bounds(a.mask, map_pos(a.qmap, min(w_first, r_last)));
  const Bounds wv_l = row_bounds(a.mask, map_pos(a.qmap, w_last));

  const int kbeg = first_ge(a.kmap, wg_f.lo);
  const int kend = min(a.lk, last_le(a.kmap, wg_l.hi) + 1);

  float m_run = NEG_INF, l_run = 0.f;
  f32x16 o[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d) o[d] = f32x16{};

  if (kbeg < kend) {
    const int jt0 = kbeg / FBK, jt1 = (kend - 1) / FBK;
    if constexpr (BF16) {
      // Software pipeline: tile jt+1 is fetched into registers while tile jt is
      // computed from LDS, then written to the other LDS buffer.
      KVStageBf16<D> stage;
      stage.load(rk, rv, kst, vst, jt0 * FBK, tid);
      stage.store(smem, smem + FBK * C::KSTR, tid);
      __syncthreads();
      for (int jt = jt0; jt <= jt1; ++jt) {
        const int cur = (jt - jt0) & 1;
        const char* sK = smem + cur * C::BUF;
        const bool more = jt < jt1;
        if (more) stage.load(rk, rv, kst, vst, (jt + 1) * FBK, tid);
        fwd_tile<D, true>(a, jt * FBK, sK, sK + FBK * C::KSTR, qf, rb, wv_f, wv_l, wave_has_rows, m_run, l_run, o,
                          l32, hf);
        if (more) {
          char* nK = smem + (cur ^ 1) * C::BUF;
          stage.store(nK, nK + FBK * C::KSTR, tid);
        }
        __syncthreads();
      }
    } else {
      for (int jt = jt0; jt <= jt1; ++jt) {
        fwd_stage_f32<D>(rk, rv, kst, vst, jt * FBK, smem, smem + FBK * C::KSTR, tid);
        __syncthreads();
        fwd_tile<D, false>(a, jt * FBK, smem, smem + FBK * C::KSTR, qf, rb, wv_f, wv_l, wave_has_rows, m_run,
                           l_run, o, l32, hf);
        __syncthreads();
      }
    }
  }

  // Epilogue: block-normalise, then store or merge into the fp32 running state.
  const float l_tot = sum_halves(l_run);
  if (!row_ok) return;
  float lse_b, inv;
  if (l_tot > 0.f) {
    lse_b = (m_run + __log2f(l_tot)) * LN2;
    inv = 1.f / l_tot;
  } else {
    lse_b = NEG_INF;
    inv = 0.f;
  }
  float* lse_p = a.lse + ((int64_t)b * a.heads + head) * a.lse_sh + row;
  float* orow = reinterpret_cast<float*>(a.out.ptr) + b * a.out.sb + (int64_t)row * a.out.st + head * a.out.sh;
  float wa = 0.f, wb = inv, lse_new = lse_b;
  if (a.mode == FWD_MERGE) {
    const float lse_old = *lse_p;
    const float mm = fmaxf(lse_old, lse_b);
    if (mm == NEG_INF) {
      wa = 0.f;
      wb = 0.f;
      lse_new = NEG_INF;
    } else {
      const float ea = expf(lse_old - mm), eb = expf(lse_b - mm);
      const float s = ea + eb;
      lse_new = mm + logf(s);
      wa = ea / s;
      wb = eb / s * inv;
    }
  }
  using TI = typename std::conditional<BF16, uint16_t, float>::type;
#pragma unroll
  for (int d = 0; d < NDB; ++d) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = d * 32 + 8 * g + 4 * hf;
      f32x4 val = {o[d][4 * g] * wb, o[d][4 * g + 1] * wb, o[d][4 * g + 2] * wb, o[d][4 * g + 3] * wb};
      if (a.mode == FWD_MERGE) {
        const f32x4 old = *reinterpret_cast<const f32x4*>(orow + d0);
        val += wa * old;
      }
      *reinterpret_cast<f32x4*>(orow + d0) = val;
      if (a.out_lowp.ptr) {
        TI* lp = reinterpret_cast<TI*>(a.out_lowp.ptr) + b * a.out_lowp.sb + (int64_t)row * a.out_lowp.st +
                 head * a.out_lowp.sh + d0;
        if constexpr (BF16) {
          const __bf16 t0 = (__bf16)val[0], t1 = (__bf16)val[1], t2 = (__bf16)val[2], t3 = (__bf16)val[3];
          const uint32_t p0 =
              (uint32_t)__builtin_bit_cast(uint16_t, t0) | ((uint32_t)__builtin_bit_cast(uint16_t, t1) << 16);
          const uint32_t p1 =
              (uint32_t)__builtin_bit_cast(uint16_t, t2) | ((uint32_t)__builtin_bit_cast(uint16_t, t3) << 16);
          *reinterpret_cast<u32x2*>(lp) = u32x2{p0, p1};
        } else {
          *reinterpret_cast<f32x4*>(lp) = val;
        }
      }
    }
  }
  if (hf == 0) *lse_p = lse_new;
}

// ============================================================================================
// Backward
// ============================================================================================

constexpr int BQB = 64;  // query rows per backward inner tile

template <int D, bool BF16>
struct BwdCfg {
  static constexpr int QSTR = BF16 ? (D + 8) * 2 : (D + 2) * 4;  // natural Q / dO rows
  static constexpr int QTSZ = BF16 ? D * 128 : 0;                // transposed Q / dO tiles
  static constexpr int SSTR = BF16 ? (BWD_BK + 8) * 2 : (BWD_BK + 2) * 4;  // dS rows
  // one buffer: Q, Q^T, dO, dO^T, then lse*log2e, delta, row lo, row hi
  static constexpr int OFF_Q = 0;
  static constexpr int OFF_QT = OFF_Q + BQB * QSTR;
  static constexpr int OFF_DO = OFF_QT + QTSZ;
  static constexpr int OFF_DOT = OFF_DO + BQB * QSTR;
  static constexpr int OFF_LSE = OFF_DOT + QTSZ;
  static constexpr int OFF_DEL = OFF_LSE + BQB * 4;
  static constexpr int OFF_LO = OFF_DEL + BQB * 4;
  static constexpr int OFF_HI = OFF_LO + BQB * 4;
  static constexpr int BUF = OFF_HI + BQB * 4;
  static constexpr int NBUF = BF16 ? 2 : 1;
  static constexpr int OFF_DS = NBUF * BUF;
  static constexpr int LDS = OFF_DS + BQB * SSTR;
};

// Per-row data of a query tile: lse (log2 units; +inf for rows without keys or
// past the end), delta, and the visible key interval.
struct RowStage {
  float l, dl;
  int lo, hi;
  __device__ __forceinline__ void load(const BwdArgs& a, const float* lse_b, const float* del_b, int r0, int tid) {
    if (tid < BQB) {
      const int r = r0 + tid;
      if (r < a.lq) {
        const float x = lse_b[r];
        l = (x == NEG_INF) ? POS_INF : x * LOG2E;
        dl = del_b[r];
        const Bounds rb = row_bounds(a.mask, map_pos(a.qmap, r));
        lo = rb.lo;
        hi = rb.hi;
      } else {
        l = POS_INF;
        dl = 0.f;
        lo = INT_BIG;
        hi = -1;
      }
    }
  }
  template <class C>
  __device__ __forceinline__ void store(char* buf, int tid) const {
    if (tid < BQB) {
      reinterpret_cast<float*>(buf + C::OFF_LSE)[tid] = l;
      reinterpret_cast<float*>(buf + C::OFF_DEL)[tid] = dl;
      reinterpret_cast<int*>(buf + C::OFF_LO)[tid] = lo;
      reinterpret_cast<int*>(buf + C::OFF_HI)[tid] = hi;
    }
  }
};

// bf16 query-tile staging (Q and dO, natural and transposed): global ->
// registers one tile ahead -> LDS.
template <int D>
struct QStageBf16 {
  static constexpr int CPR = D / 8;
  static constexpr int ITEMS = (BQB / 4) * CPR;  // (4 rows x 8 d) items
  u32x4 q[4], g[4];
  RowStage rows;

  __device__ __forceinline__ void load(const BwdArgs& a, Rsrc rq, Rsrc rdo, uint32_t qst, uint32_t dst,
                                       const float* lse_b, const float* del_b, int r0, int tid) {
    if (tid < ITEMS) {
      const int c = tid % CPR, rq4 = tid / CPR;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        q[i] = bload16(rq, (uint32_t)(r0 + 4 * rq4 + i) * qst + c * 16);
        g[i] = bload16(rdo, (uint32_t)(r0 + 4 * rq4 + i) * dst + c * 16);
      }
    }
    rows.load(a, lse_b, del_b, r0, tid);
  }
  __device__ __forceinline__ static void put(const u32x4* x, char* sN, char* sT, int c, int rq4) {
    constexpr int QSTR = BwdCfg<D, true>::QSTR;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(sN + (4 * rq4 + i) * QSTR + c * 16) = x[i];
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      const int e = dd >> 1;
      uint32_t w0, w1;
      if (dd & 1) {
        w0 = (x[0][e] >> 16) | (x[1][e] & 0xffff0000u);
        w1 = (x[2][e] >> 16) | (x[3][e] & 0xffff0000u);
      } else {
        w0 = (x[0][e] & 0xffffu) | (x[1][e] << 16);
        w1 = (x[2][e] & 0xffffu) | (x[3][e] << 16);
      }
      *reinterpret_cast<u32x2*>(sT + tr_off(8 * c + dd, 4 * rq4)) = u32x2{w0, w1};
    }
  }
  __device__ __forceinline__ void store(char* buf, int tid) const {
    using C = BwdCfg<D, true>;
    if (tid < ITEMS) {
      const int c = tid % CPR, rq4 = tid / CPR;
      put(q, buf + C::OFF_Q, buf + C::OFF_QT, c, rq4);
      put(g, buf + C::OFF_DO, buf + C::OFF_DOT, c, rq4);
    }
    rows.store<C>(buf, tid);
  }
};

template <int D>
__device__ __forceinline__ void bwd_stage_f32(const BwdArgs& a, Rsrc rq, Rsrc rdo, uint32_t qst, uint32_t dst,
                                              const float* lse_b, const float* del_b, int r0, char* buf, int tid) {
  using C = BwdCfg<D, false>;
  constexpr int CPR = D / 4;
  constexpr int ITEMS = BQB * CPR;
#pragma unroll 4
  for (int it = tid; it < ITEMS; it += NT) {
    const int r = it / CPR, c = it % CPR;
    const f32x4 x = bload16f(rq, (uint32_t)(r0 + r) * qst + c * 16);
    const f32x4 y = bload16f(rdo, (uint32_t)(r0 + r) * dst + c * 16);
    float* dq = reinterpret_cast<float*>(buf + C::OFF_Q + r * C::QSTR) + c * 4;
    float* dd = reinterpret_cast<float*>(buf + C::OFF_DO + r * C::QSTR) + c * 4;
    *reinterpret_cast<float2*>(dq) = make_float2(x[0], x[1]);
    *reinterpret_cast<float2*>(dq + 2) = make_float2(x[2], x[3]);
    *reinterpret_cast<float2*>(dd) = make_float2(y[0], y[1]);
    *reinterpret_cast<float2*>(dd + 2) = make_float2(y[2], y[3]);
  }
  RowStage rows;
  rows.load(a, lse_b, del_b, r0, tid);
  rows.store<C>(buf, tid);
}

template <int D, bool BF16>
__global__ __launch_bounds__(NT, 1) void bwd_kernel(BwdArgs a) {
  using C = BwdCfg<D, BF16>;
  constexpr int NDB = D / 32;
  constexpr int ESZ = BF16 ? 2 : 4;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];
  char* sDS = smem + C::OFF_DS;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int logical = xcd_logical(blockIdx.x, gridDim.x);
  const int kt = logical % a.n_ktiles;  // earliest (heaviest causal) key tiles first
  const int bh = logical / a.n_ktiles;
  const int head = bh % a.heads, b = bh / a.heads;

  const char* qbase = reinterpret_cast<const char*>(a.q.ptr) + (b * a.q.sb + head * a.q.sh) * ESZ;
  const char* kbase = reinterpret_cast<const char*>(a.k.ptr) + (b * a.k.sb + head * a.k.sh) * ESZ;
  const char* vbase = reinterpret_cast<const char*>(a.v.ptr) + (b * a.v.sb + head * a.v.sh) * ESZ;
  const char* dobase = reinterpret_cast<const char*>(a.dout.ptr) + (b * a.dout.sb + head * a.dout.sh) * ESZ;
  const Rsrc rq = make_rsrc(qbase, slice_bytes(a.lq, a.q.st, ESZ, D));
  const Rsrc rk = make_rsrc(kbase, slice_bytes(a.lk, a.k.st, ESZ, D));
  const Rsrc rv = make_rsrc(vbase, slice_bytes(a.lk, a.v.st, ESZ, D));
  const Rsrc rdo = make_rsrc(dobase, slice_bytes(a.lq, a.dout.st, ESZ, D));
  const uint32_t qst = (uint32_t)(a.q.st * ESZ), kst = (uint32_t)(a.k.st * ESZ);
  const uint32_t vst = (uint32_t)(a.v.st * ESZ), dst = (uint32_t)(a.dout.st * ESZ);
  const float* lse_b = a.lse + ((int64_t)b * a.heads + head) * a.lse_sh;
  const float* del_b = a.delta + ((int64_t)b * a.heads + head) * a.lse_sh;
  float* dqb = reinterpret_cast<float*>(a.dq.ptr) + b * a.dq.sb + head * a.dq.sh;

  const int k_first = kt * BWD_BK;
  const int k_last = min(a.lk, k_first + BWD_BK) - 1;
  const int kw0 = k_first + 32 * w;
  const int kw_last = min(k_last, kw0 + 31);
  const bool wave_has_keys = kw0 <= k_last;
  const int key = kw0 + l32;
  const bool key_ok = key <= k_last;
  const int kpos = map_pos(a.kmap, min(key, k_last));

  // Key/value fragments (B operands of S = Q K^T and dP = dO V^T).
  constexpr int NKF = BF16 ? D / 16 : D / 2;
  typedef typename std::conditional<BF16, bf16x8, float>::type KF;
  KF kf[NKF], vf[NKF];
  if constexpr (BF16) {
#pragma unroll
    for (int c = 0; c < NKF; ++c) {
      kf[c] = __builtin_bit_cast(bf16x8, bload16(rk, (uint32_t)key * kst + (16 * c + 8 * hf) * 2));
      vf[c] = __builtin_bit_cast(bf16x8, bload16(rv, (uint32_t)key * vst + (16 * c + 8 * hf) * 2));
    }
  } else {
#pragma unroll
    for (int c4 = 0; c4 < D / 4; ++c4) {
      const f32x4 x = bload16f(rk, (uint32_t)key * kst + 16 * c4);
      const f32x4 y = bload16f(rv, (uint32_t)key * vst + 16 * c4);
      kf[2 * c4] = hf ? x[1] : x[0];
      kf[2 * c4 + 1] = hf ? x[3] : x[2];
      vf[2 * c4] = hf ? y[1] : y[0];
      vf[2 * c4 + 1] = hf ? y[3] : y[2];
    }
  }

  // dQ assignment: (query block, d block) pairs of the 64 x D dQ tile.
  constexpr int PAIRS = 2 * NDB / 4;  // per wave: 2 for D=128, 1 for D=64
  const int dq_db = (D == 128) ? w : (w & 1);
  const int dq_qb0 = (D == 128) ? 0 : (w >> 1);
  const int dcol = dq_db * 32 + l32;
  // K^T fragments for dQ = dS K (bf16: 8 consecutive keys of one d per lane).
  bf16x8 ktf[BF16 ? BWD_BK / 16 : 1];
  if constexpr (BF16) {
#pragma unroll
    for (int jj = 0; jj < BWD_BK / 16; ++jj)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        ktf[jj][i] = __builtin_bit_cast(__bf16, bload2(rk, (uint32_t)(k_first + 16 * jj + 8 * hf + i) * kst + dcol * 2));
  }

  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d) {
    dk[d] = f32x16{};
    dv[d] = f32x16{};
  }

  // Query rows that can see any key of this tile.
  const Bounds cf = col_bounds(a.mask, map_pos(a.kmap, k_first));
  const Bounds cl = col_bounds(a.mask, map_pos(a.kmap, k_last));
  const int rbeg = first_ge(a.qmap, cf.lo);
  const int rend = min(a.lq, last_le(a.qmap, cl.hi) + 1);
  const int kwmin = map_pos(a.kmap, min(kw0, k_last)), kwmax = map_pos(a.kmap, kw_last);
  const float sl2 = a.scale_log2;

  if (rbeg < rend) {
    const int qt0 = rbeg / BQB, qt1 = (rend - 1) / BQB;
    QStageBf16<D> stage;
    if constexpr (BF16) {
      stage.load(a, rq, rdo, qst, dst, lse_b, del_b, qt0 * BQB, tid);
      stage.store(smem, tid);
      __syncthreads();
    }
    for (int qt = qt0; qt <= qt1; ++qt) {
      const int r0 = qt * BQB;
      const int nrows = min(a.lq - r0, BQB);
      const int cur = BF16 ? ((qt - qt0) & 1) : 0;
      char* buf = smem + cur * C::BUF;
      const bool more = qt < qt1;
      if constexpr (BF16) {
        if (more) stage.load(a, rq, rdo, qst, dst, lse_b, del_b, (qt + 1) * BQB, tid);
      } else {
        bwd_stage_f32<D>(a, rq, rdo, qst, dst, lse_b, del_b, r0, buf, tid);
        __syncthreads();
      }
      const char* sQ = buf + C::OFF_Q;
      const char* sQt = buf + C::OFF_QT;
      const char* sDO = buf + C::OFF_DO;
      const char* sDOt = buf + C::OFF_DOT;
      const float* sLse = reinterpret_cast<const float*>(buf + C::OFF_LSE);
      const float* sDel = reinterpret_cast<const float*>(buf + C::OFF_DEL);
      const int* sLo = reinterpret_cast<const int*>(buf + C::OFF_LO);
      const int* sHi = reinterpret_cast<const int*>(buf + C::OFF_HI);

      const int lo_f = sLo[0], hi_f = sHi[0], lo_l = sLo[nrows - 1], hi_l = sHi[nrows - 1];
      const bool wave_empty = !wave_has_keys || kwmax < lo_f || kwmin > hi_l;
      const bool wave_full = (kw0 + 32 <= a.lk) && kwmin >= lo_l && kwmax <= hi_f;

#pragma unroll
      for (int qbk = 0; qbk < 2; ++qbk) {
        if (wave_empty) {
          // A wave with nothing visible still provides its (zero) dS columns.
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int q = qbk * 32 + reg_row(v, hf);
            if constexpr (BF16)
              *reinterpret_cast<uint16_t*>(sDS + q * C::SSTR + (32 * w + l32) * 2) = 0;
            else
              *reinterpret_cast<float*>(sDS + q * C::SSTR + (32 * w + l32) * 4) = 0.f;
          }
          continue;
        }
        // S = Q K^T (rows permuted) and dP = dO V^T.
        f32x16 s = f32x16{}, dp = f32x16{};
        if constexpr (BF16) {
          const char* qr = sQ + (qbk * 32 + row_perm(l32)) * C::QSTR + hf * 16;
          const char* dr = sDO + (qbk * 32 + row_perm(l32)) * C::QSTR + hf * 16;
#pragma unroll
          for (int c = 0; c < D / 16; ++c) s = mfma_bf16(ld_bf16x8(qr + c * 32), kf[c], s);
#pragma unroll
          for (int c = 0; c < D / 16; ++c) dp = mfma_bf16(ld_bf16x8(dr + c * 32), vf[c], dp);
        } else {
          const float* qr = reinterpret_cast<const float*>(sQ + (qbk * 32 + row_perm(l32)) * C::QSTR) + hf;
          const float* dr = reinterpret_cast<const float*>(sDO + (qbk * 32 + row_perm(l32)) * C::QSTR) + hf;
#pragma unroll
          for (int t = 0; t < D / 2; ++t) s = mfma_f32(qr[2 * t], kf[t], s);
#pragma unroll
          for (int t = 0; t < D / 2; ++t) dp = mfma_f32(dr[2 * t], vf[t], dp);
        }
        // P = exp2(S*scale*log2e - lse*log2e); dS = P * (dP - delta).
        f32x16 p, ds;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int q = qbk * 32 + reg_row(v, hf);
          float e = ex2(__builtin_fmaf(s[v], sl2, -sLse[q]));
          if (!wave_full) {
            const bool ok = key_ok && kpos >= sLo[q] && kpos <= sHi[q];
            e = ok ? e : 0.f;
          }
          p[v] = e;
          ds[v] = e * (dp[v] - sDel[q]);
        }
        // dV^T += dO^T P and dK^T += Q^T dS (K-dim = query rows).
        if constexpr (BF16) {
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            bf16x8 pb, sb;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              pb[i] = (__bf16)p[8 * u + i];
              sb[i] = (__bf16)ds[8 * u + i];
            }
            const int qcol = qbk * 32 + 16 * u + 8 * hf;
#pragma unroll
            for (int d = 0; d < NDB; ++d) {
              dv[d] = mfma_bf16(ld_bf16x8(sDOt + tr_off(d * 32 + l32, qcol)), pb, dv[d]);
              dk[d] = mfma_bf16(ld_bf16x8(sQt + tr_off(d * 32 + l32, qcol)), sb, dk[d]);
            }
          }
        } else {
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            const int q = qbk * 32 + reg_row(t, hf);
            const float* dor = reinterpret_cast<const float*>(sDO + q * C::QSTR) + l32;
            const float* qr = reinterpret_cast<const float*>(sQ + q * C::QSTR) + l32;
#pragma unroll
            for (int d = 0; d < NDB; ++d) {
              dv[d] = mfma_f32(dor[d * 32], p[t], dv[d]);
              dk[d] = mfma_f32(qr[d * 32], ds[t], dk[d]);
            }
          }
        }
        // dS -> LDS [query][key] for the dQ product.
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int q = qbk * 32 + reg_row(v, hf);
          if constexpr (BF16)
            *reinterpret_cast<__bf16*>(sDS + q * C::SSTR + (32 * w + l32) * 2) = (__bf16)ds[v];
          else
            *reinterpret_cast<float*>(sDS + q * C::SSTR + (32 * w + l32) * 4) = ds[v];
        }
      }
      __syncthreads();

      // dQ[tile rows] += scale * dS K  (M = query rows, N = d, K-dim = this tile's keys).
#pragma unroll
      for (int pi = 0; pi < PAIRS; ++pi) {
        const int qbk = dq_qb0 + pi;
        f32x16 acc = f32x16{};
        if constexpr (BF16) {
          const char* sr = sDS + (qbk * 32 + l32) * C::SSTR + hf * 16;
#pragma unroll
          for (int jj = 0; jj < BWD_BK / 16; ++jj) acc = mfma_bf16(ld_bf16x8(sr + jj * 32), ktf[jj], acc);
        } else {
          const float* sr = reinterpret_cast<const float*>(sDS + (qbk * 32 + l32) * C::SSTR) + hf;
#pragma unroll 8
          for (int t = 0; t < BWD_BK / 2; ++t)
            acc = mfma_f32(sr[2 * t], bload4f(rk, (uint32_t)(k_first + 2 * t + hf) * kst + dcol * 4), acc);
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int q = qbk * 32 + 8 * (v >> 2) + 4 * hf + (v & 3);
          const int r = r0 + q;
          if (r < a.lq) atomicAdd(dqb + (int64_t)r * a.dq.st + dcol, acc[v] * a.scale);
        }
      }
      if constexpr (BF16) {
        if (more) stage.store(smem + (cur ^ 1) * C::BUF, tid);
      }
      __syncthreads();
    }
  }

  // Epilogue: dK += scale * dK^T, dV += dV^T (fp32 read-modify-write; this
  // workgroup owns these key rows for the whole launch).
  if (!key_ok) return;
  float* dkr = reinterpret_cast<float*>(a.dk.ptr) + b * a.dk.sb + (int64_t)key * a.dk.st + head * a.dk.sh;
  float* dvr = reinterpret_cast<float*>(a.dv.ptr) + b * a.dv.sb + (int64_t)key * a.dv.st + head * a.dv.sh;
#pragma unroll
  for (int d = 0; d < NDB; ++d)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = d * 32 + 8 * g + 4 * hf;
      f32x4 x = *reinterpret_cast<const f32x4*>(dkr + d0);
      f32x4 y = *reinterpret_cast<const f32x4*>(dvr + d0);
      x += a.scale * f32x4{dk[d][4 * g], dk[d][4 * g + 1], dk[d][4 * g + 2], dk[d][4 * g + 3]};
      y += f32x4{dv[d][4 * g], dv[d][4 * g + 1], dv[d][4 * g + 2], dv[d][4 * g + 3]};
      *reinterpret_cast<f32x4*>(dkr + d0) = x;
      *reinterpret_cast<f32x4*>(dvr + d0) = y;
    }
}

// ============================================================================================
// bf16 tiles in LDS.  Every tile is stored in its natural [row][D] layout with
// the 16-byte chunks of each row XOR-swizzled, filled by direct buffer->LDS
// loads (no registers, no VALU) and read two ways:
//  * as MFMA rows: lane (row, half) reads 16 bytes = 8 consecutive elements of
//    one row (A operand of S^T = K Q^T, S = Q K^T, dP = dO V^T, ...);
//  * transposed, with the LDS transpose read: in each 16-lane group lane i
//    receives element (i mod 4) of the 8-byte chunk addressed by group lane
//    4r + i/4, for r = 0..3.  Pointing group lane j at row key0 + j/4, columns
//    4(j mod 4).. of the group's 16 columns gives every lane 4 consecutive rows
//    of ONE column; two such reads form an MFMA operand whose K-dim runs over
//    rows (V^T for O^T += V^T P^T, K^T for dQ, Q^T / dO^T for dK / dV).
// The swizzle keeps both read patterns free of LDS bank conflicts: the 16 rows
// a 16-lane set reads as MFMA rows hit 16 distinct chunk positions, and the
// 4 rows x 2 chunks of a transposed read hit 8 distinct positions.
// ============================================================================================

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;

// Chunk swizzle of a natural [rows][D] bf16 LDS tile: 16-byte chunk c of row r
// sits at chunk position c ^ swz(r).  For D = 128 it is a linear map of the row
// bits 0..3 (row bit b flips the position bits of mask {6, 10, 8, 13}[b]),
// chosen so that on gfx950's 64-bank LDS both access patterns of the kernels
// are free of bank conflicts: 16-byte row reads of 32 rows (row_perm order),
// served 16 lanes at a time, and the transposed 8-byte reads of 8-row column
// strips, served 32 lanes at a time (checked with the SQ_LDS_BANK_CONFLICT
// counter).  It depends on the row modulo 16 only.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128)
    return (6 & -(r & 1)) ^ (10 & -((r >> 1) & 1)) ^ (8 & -((r >> 2) & 1)) ^ (13 & -((r >> 3) & 1));
  else return (r >> 1) & 7;
}
// Byte offset of 16-byte chunk `chunk` of row `row` in a swizzled [rows][D] bf16 tile.
template <int D>
__device__ __forceinline__ int nat_off(int row, int chunk) {
  return row * (D * 2) + ((chunk ^ swz<D>(row)) << 4);
}
__device__ __forceinline__ u32x2 tr16(const char* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p)));
}
// MFMA operand from a transposed read: rows key0 .. key0+7 (key0 already holds
// the lane half's offset) of column 32*db + (lane mod 32).
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const char* tile, int key0, int db, int lane) {
  const int j = lane & 15, g1 = (lane >> 4) & 1;
  const int colb = 2 * (32 * db + 16 * g1 + 4 * (j & 3));
  const int chunk = colb >> 4, within = colb & 15;
  const u32x2 lo = tr16(tile + nat_off<D>(key0 + (j >> 2), chunk) + within);
  const u32x2 hi = tr16(tile + nat_off<D>(key0 + 4 + (j >> 2), chunk) + within);
  return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}
// 8 consecutive elements (16-byte chunk 2c + hf) of row `row`: an MFMA row operand.
template <int D>
__device__ __forceinline__ bf16x8 row_operand(const char* tile, int row, int c, int hf) {
  return ld_bf16x8(tile + nat_off<D>(row, 2 * c + hf));
}
// Direct buffer->LDS copy of rows [r0, r0 + ROWS) of a [rows][D] bf16 slice into
// a swizzled tile; wave w of NWAVES moves rows [w*ROWS/NWAVES, (w+1)*ROWS/NWAVES).  Rows past the
// slice read as zeros (buffer range check).  `w` must be wave-uniform.
template <int D, int ROWS, int NWAVES = 4>
__device__ __forceinline__ void dma_tile(Rsrc rs, uint32_t st, int r0, char* tile, int w, int lane) {
  constexpr int RPI = 1024 / (2 * D);  // rows per instruction (64 lanes x 16 bytes)
  constexpr int CPR = (2 * D) / 16;    // chunks per row
  constexpr int RPW = ROWS / NWAVES;   // rows per wave
  static_assert(RPW % RPI == 0, "tile rows must split evenly over the waves");
#pragma unroll
  for (int i = 0; i < RPW / RPI; ++i) {
    const int rbase = w * RPW + i * RPI;
    const int row = rbase + lane / CPR;
    const int c = (lane % CPR) ^ swz<D>(row);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(tile + rbase * 2 * D), 16,
                                             (uint32_t)(r0 + row) * st + c * 16, 0, 0, 0);
  }
}
// The same copy with the per-lane part of every offset derived from two
// registers: the swizzle is linear in the row bits and every instruction's
// first row rbase is a multiple of the rows it covers, so its chunk is
// cx ^ swz(rbase) (wave-uniform) with cx = (lane mod CPR) ^ swz(lane / CPR),
// and the row part splits into lane_row * st plus a wave-uniform scalar offset.
// `cx16` = 16 * cx and `lrow_st` = (lane / CPR) * st come from dma_lane_parts().
template <int D>
__device__ __forceinline__ void dma_lane_parts(int lane, uint32_t st, uint32_t& cx16, uint32_t& lrow_st) {
  constexpr int CPR = (2 * D) / 16;
  cx16 = (uint32_t)(((lane % CPR) ^ swz<D>(lane / CPR)) << 4);
  lrow_st = (uint32_t)(lane / CPR) * st;
}
template <int D, int ROWS, int NWAVES = 4>
__device__ __forceinline__ void dma_tile_lean(Rsrc rs, uint32_t st, int r0, char* tile, int w, uint32_t cx16,
                                              uint32_t lrow_st) {
  constexpr int RPI = 1024 / (2 * D);
  constexpr int RPW = ROWS / NWAVES;
  static_assert(RPW % RPI == 0, "wave rows must split into whole instructions");
#pragma unroll
  for (int i = 0; i < RPW / RPI; ++i) {
    const int rbase = w * RPW + i * RPI;  // wave-uniform, a multiple of RPI
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(tile + rbase * 2 * D), 16,
                                             lrow_st + (cx16 ^ (uint32_t)(swz<D>(rbase) << 4)),
                                             (uint32_t)(r0 + rbase) * st, 0, 0);
  }
}
// Wait for this wave's outstanding global/buffer loads (including buffer->LDS).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// Wait until at most N of this wave's vector-memory operations are outstanding
// (they complete in issue order), leaving the newest N in flight.
template <int N>
__device__ __forceinline__ void wait_vmem_keep() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
// Workgroup barrier without __syncthreads()' release fence, which waits for
// every outstanding vector-memory operation of the wave, buffer->LDS copies
// still in flight included.  The caller makes its own LDS writes complete with
// explicit waits before it; the asm's memory clobber keeps the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void barrier_keep_vmem() { asm volatile("s_barrier" ::: "memory"); }
// Direct buffer->LDS copy of 64 consecutive fp32 values (one per lane).
__device__ __forceinline__ void dma_f32x64(Rsrc rs, int first, char* dst, int lane) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)dst, 4, (uint32_t)(first + lane) * 4, 0, 0, 0);
}

// ============================================================================================
// bf16 forward, software-pipelined over tiles of 64 keys: while a wave turns
// S of tile j into P (exponentials), it already issues the MFMAs of S for
// tile j + 1, so that the matrix unit has work during the softmax; P V is
// added into O after a barrier in the middle of the step.  K tiles are
// therefore DMA'd two tiles ahead and V tiles one ahead, each into the other
// of two LDS buffers; a V tile has one and a half steps to land, a K tile one.
// ============================================================================================

template <int D>
struct FwdB {
  static constexpr int TILE = FBK * D * 2;  // bytes of one K (or V) tile
};

template <int D>
__global__ __launch_bounds__(NT, 2) void fwd_kernel_bf16(FwdArgs ap) {
  FwdArgs a = ap;
  int bid = (int)blockIdx.x, nblk = (int)gridDim.x;
  if (ap.g.n) fwd_piece(ap, a, bid, nblk);
  using C = FwdB<D>;
  constexpr int NDB = D / 32;
  // Two K and two V buffers, four LDS objects: every read addresses one of
  // them through one register plus an immediate, which lets the compiler see
  // that a read does not touch the buffer a DMA is filling (it would
  // otherwise wait for every copy in flight before the read).
  __shared__ __attribute__((aligned(16))) char k_buf0[C::TILE];
  __shared__ __attribute__((aligned(16))) char k_buf1[C::TILE];
  __shared__ __attribute__((aligned(16))) char v_buf0[C::TILE];
  __shared__ __attribute__((aligned(16))) char v_buf1[C::TILE];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int logical = xcd_logical(bid, nblk);
  const int qt = a.n_qtiles - 1 - logical % a.n_qtiles;  // latest (heaviest causal) tiles first
  const int bh = logical / a.n_qtiles;
  if (bh >= a.heads * a.batch) return;  // a grouped launch's padding block
  const int head = bh % a.heads, b = bh / a.heads;

  const int r_first = qt * FWD_BQ;
  const int r_last = min(a.lq, r_first + FWD_BQ) - 1;
  const int w_first = r_first + 32 * w;
  const int w_last = min(r_last, w_first + 31);
  const bool wave_has_rows = w_first <= r_last;
  const int row = w_first + l32;
  const bool row_ok = row <= r_last;

  const char* qbase = reinterpret_cast<const char*>(a.q.ptr) + (b * a.q.sb + head * a.q.sh) * 2;
  const char* kbase = reinterpret_cast<const char*>(a.k.ptr) + (b * a.k.sb + head * a.k.sh) * 2;
  const char* vbase = reinterpret_cast<const char*>(a.v.ptr) + (b * a.v.sb + head * a.v.sh) * 2;
  const Rsrc rq = make_rsrc(qbase, slice_bytes(a.lq, a.q.st, 2, D));
  const Rsrc rk = make_rsrc(kbase, slice_bytes(a.lk, a.k.st, 2, D));
  const Rsrc rv = make_rsrc(vbase, slice_bytes(a.lk, a.v.st, 2, D));
  const uint32_t qst = (uint32_t)(a.q.st * 2), kst = (uint32_t)(a.k.st * 2), vst = (uint32_t)(a.v.st * 2);

  const Bounds wg_f = row_bounds(a.mask, map_pos(a.qmap, r_first));
  const Bounds wg_l = row_bounds(a.mask, map_pos(a.qmap, r_last));
  const int kbeg = first_ge(a.kmap, wg_f.lo);
  const int kend = min(a.lk, last_le(a.kmap, wg_l.hi) + 1);
  // No row of this workgroup sees any key of the block (positions increase with
  // the row, and so do both ends of a row's visible interval): merging an empty
  // block leaves out and lse as they are, so such a workgroup touches nothing
  // unless it must write the first result or the low-precision copy.
  if (kbeg >= kend && a.mode == FWD_MERGE && a.out_lowp.ptr == nullptr) return;

  bf16x8 qf[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c)
    qf[c] = __builtin_bit_cast(bf16x8, bload16(rq, (uint32_t)row * qst + (16 * c + 8 * hf) * 2));

  const Bounds rb = row_bounds(a.mask, map_pos(a.qmap, min(row, r_last)));
  const Bounds wv_f = row_bounds(a.mask, map_pos(a.qmap, min(w_first, r_last)));
  const Bounds wv_l = row_bounds(a.mask, map_pos(a.qmap, w_last));
  const float sl2 = a.scale_log2;
  // Key positions increase with the key index, so this lane's row sees the
  // keys of one index interval, [ja, ja + jspan] (ja far past every key when
  // it sees none): a tile that the wave's rows do not all see whole is masked
  // with one unsigned compare per score.
  int ja = first_ge(a.kmap, rb.lo), jspan = 0;
  {
    const int jb = min(a.lk - 1, last_le(a.kmap, rb.hi));
    if (jb < ja || !wave_has_rows) ja = 1 << 30;
    else jspan = jb - ja;
  }

  float m_run = NEG_INF, l_run = 0.f, m_use = 0.f;
  f32x16 o[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d) o[d] = f32x16{};

  // Per-lane byte offsets of the LDS operand reads within a tile: K row krow
  // (row_perm order), 16-byte chunk 2c + hf (row krow + 32 sits 32 rows, an
  // immediate, further: the swizzle depends on the row modulo 16 only); and
  // the transposed V reads of key rows 8*hf + (j >> 2) + 4*hi (j = lane mod 16)
  // at column 32*d + 16*g1 + 4*(j & 3), g1 = bit 4 of the lane (key rows 16*m
  // further are immediates too).
  const int krow = row_perm(l32);
  int offK[D / 16], offV[NDB][2];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) offK[c] = nat_off<D>(krow, 2 * c + hf);
  {
    const int j = lane & 15, g1 = (lane >> 4) & 1;
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int colb = 2 * (32 * d + 16 * g1 + 4 * (j & 3));
        offV[d][hi] = nat_off<D>(8 * hf + (j >> 2) + 4 * hi, colb >> 4) + (colb & 15);
      }
  }
  // S^T of one tile (keys x this wave's rows) for the two 32-key halves, the
  // two MFMA chains interleaved.
  auto s_tile = [&](const char* sK, f32x16* st) {
    st[0] = f32x16{};
    st[1] = f32x16{};
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      st[0] = mfma_bf16(ld_bf16x8(sK + offK[c]), qf[c], st[0]);
      st[1] = mfma_bf16(ld_bf16x8(sK + offK[c] + 32 * 2 * D), qf[c], st[1]);
    }
  };
  // Visibility of tile jt's S^T for this wave's rows (-inf where a query row
  // does not see a key), then the running maximum: O and the row sum are
  // rescaled only when a row's maximum grows by more than RESCALE_TH (so that
  // every P stays below 2^RESCALE_TH); the result is exact either way.
  auto mask_max = [&](int jt, f32x16* st) {
    const int j0 = jt * FBK;
    const int jl = min(a.lk, j0 + FBK) - 1;
    const int kmin = map_pos(a.kmap, j0), kmax = map_pos(a.kmap, jl);
    const bool vis = wave_has_rows && kmax >= wv_f.lo && kmin <= wv_l.hi;
    const bool full = vis && (j0 + FBK <= a.lk) && kmin >= wv_l.lo && kmax <= wv_f.hi;
    if (!full) {
      // key index of score (c2, v) = j0 + 8 * hf + 32 * c2 + (v < 8 ? v : v + 8)
      const int t = j0 + 8 * hf - ja;
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const bool ok = (uint32_t)(t + 32 * c2 + (v < 8 ? v : v + 8)) <= (uint32_t)jspan;
          st[c2][v] = ok ? st[c2][v] : NEG_INF;
        }
    }
    float mx = NEG_INF;
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, st[c2][v]);
    mx = max_halves(mx) * sl2;
    const bool grow = mx > m_run + RESCALE_TH;
    if (__any(grow)) {
      const float m_new = grow ? mx : m_run;
      const float alpha = (m_new == m_run) ? 1.f : ex2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < NDB; ++d) o[d] *= alpha;
      m_run = m_new;
    }
    m_use = (m_run == NEG_INF) ? 0.f : m_run;
  };
  // P = exp2(S * scale*log2(e) - m) for the finished tile as bf16 operands, and
  // its row sums; then, once the V tile has landed, O^T += V^T P^T (V^T through
  // the transposed read of the natural V tile).
  auto p_only = [&](f32x16* st, bf16x8* pb) {
    float rs = 0.f;
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = ex2(__builtin_fmaf(st[c2][v], sl2, -m_use));
        st[c2][v] = p;
        rs += p;
      }
    l_run += rs;
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int q = 0; q < 8; ++q) pb[2 * c2 + u][q] = (__bf16)st[c2][8 * u + q];
  };
  auto pv_only = [&](const bf16x8* pb, const char* sV) {
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int kb0 = (c2 * 32 + 16 * u) * 2 * D;
#pragma unroll
        for (int d = 0; d < NDB; ++d) {
          const u32x2 lo = tr16(sV + offV[d][0] + kb0), hi = tr16(sV + offV[d][1] + kb0);
          o[d] = mfma_bf16(__builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]}), pb[2 * c2 + u], o[d]);
        }
      }
  };

  if (kbeg < kend) {
    const int jt0 = kbeg / FBK, jt1 = (kend - 1) / FBK;
    dma_tile<D, FBK>(rk, kst, jt0 * FBK, k_buf0, w, lane);
    dma_tile<D, FBK>(rv, vst, jt0 * FBK, v_buf0, w, lane);
    if (jt0 < jt1) dma_tile<D, FBK>(rk, kst, (jt0 + 1) * FBK, k_buf1, w, lane);
    wait_vmem();
    __syncthreads();
    f32x16 sa[2], sb[2];
    s_tile(k_buf0, sa);
    mask_max(jt0, sa);
    __syncthreads();  // K buffer 0 is refilled below
    // Tile jt is finished from `cur` while S of tile jt + 1 goes into `nxt`.
    // On the last tile the S MFMAs read a stale buffer and are discarded, so
    // that the work between the barriers has no branch.
    uint32_t cx16, lk_st, lv_st;
    dma_lane_parts<D>(lane, kst, cx16, lk_st);
    dma_lane_parts<D>(lane, vst, cx16, lv_st);
    // Tile jt (even offset from jt0: K of jt + 1 in k_buf1, V of jt in v_buf0;
    // odd: the other two) while V of jt + 1 and K of jt + 2 are fetched.
    auto step = [&](int jt, f32x16* cur, f32x16* nxt, const char* sKn, const char* sV, char* dV, char* dK) {
      // The copies' per-lane offsets do not change over the loop: held in
      // registers (8), they cost no VALU issue slots per tile, which the
      // exponentials and the MFMAs compete for.
      const uint32_t c16 = cx16, lks = lk_st, lvs = lv_st;
      // Past the end the last tile is fetched again into the free buffer, so
      // that the copies stay in the block of MFMAs; there they are spread one
      // per MFMA (all of a workgroup's copies at once queue up in the
      // vector-memory path and hold the waves that issue them).  K first: at
      // the end of the step only this K copy is waited for, while the V copy
      // has until the middle of the next step (the last copy of a step to land
      // is what a wave waits for).
      dma_tile_lean<D, FBK>(rk, kst, min(jt + 2, jt1) * FBK, dK, w, c16, lks);
      dma_tile_lean<D, FBK>(rv, vst, min(jt + 1, jt1) * FBK, dV, w, c16, lvs);
      s_tile(sKn, nxt);
      bf16x8 pb[4];
      p_only(cur, pb);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);    // K operands of the first two k-steps
#pragma unroll
      for (int g = 0; g < 2 * (FBK / (1024 / (2 * D))) / 4; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one buffer->LDS copy
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // operands two k-steps ahead
      }
      // V of this tile (copied during the previous step): every copy issued
      // before this step's two has landed, in every wave after the barrier
      wait_vmem_keep<2 * (FBK / 4) / (1024 / (2 * D))>();
      barrier_keep_vmem();
      pv_only(pb, sV);
      if (jt + 1 <= jt1) mask_max(jt + 1, nxt);
      wait_vmem_keep<(FBK / 4) / (1024 / (2 * D))>();     // this step's K copy, not its V copy
      barrier_keep_vmem();
    };
    for (int jt = jt0; jt <= jt1; jt += 2) {
      step(jt, sa, sb, k_buf1, v_buf0, v_buf1, k_buf0);
      if (jt + 1 <= jt1) step(jt + 1, sb, sa, k_buf0, v_buf1, v_buf0, k_buf1);
    }
  }

  wait_vmem();  // the last V copy: no copy into LDS may outlive the workgroup
  const float l_tot = sum_halves(l_run);
  if (!row_ok) return;
  float lse_b, inv;
  if (l_tot > 0.f) {
    lse_b = (m_run + __log2f(l_tot)) * LN2;
    inv = 1.f / l_tot;
  } else {
    lse_b = NEG_INF;
    inv = 0.f;
  }
  float* lse_p = a.lse + ((int64_t)b * a.heads + head) * a.lse_sh + row;
  float* orow = reinterpret_cast<float*>(a.out.ptr) + b * a.out.sb + (int64_t)row * a.out.st + head * a.out.sh;
  // The running output's 16 vectors of this lane are all read before any
  // store, so that their reads are in flight together (read one by one
  // between the stores, each waited for its own round trip).
  f32x4 prev[NDB][4];
  float lse_old = 0.f;
  if (a.mode == FWD_MERGE) {
    lse_old = *lse_p;
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) prev[d][g] = *reinterpret_cast<const f32x4*>(orow + d * 32 + 8 * g + 4 * hf);
  }
  float wa = 0.f, wb = inv, lse_new = lse_b;
  if (a.mode == FWD_MERGE) {
    const float mm = fmaxf(lse_old, lse_b);
    if (mm == NEG_INF) {
      wa = 0.f;
      wb = 0.f;
      lse_new = NEG_INF;
    } else {
      const float ea = expf(lse_old - mm), eb = expf(lse_b - mm);
      const float s = ea + eb;
      lse_new = mm + logf(s);
      wa = ea / s;
      wb = eb / s * inv;
    }
  }
#pragma unroll
  for (int d = 0; d < NDB; ++d) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = d * 32 + 8 * g + 4 * hf;
      f32x4 val = {o[d][4 * g] * wb, o[d][4 * g + 1] * wb, o[d][4 * g + 2] * wb, o[d][4 * g + 3] * wb};
      if (a.mode == FWD_MERGE) val += wa * prev[d][g];
      *reinterpret_cast<f32x4*>(orow + d0) = val;
      if (a.out_lowp.ptr) {
        uint16_t* lp = reinterpret_cast<uint16_t*>(a.out_lowp.ptr) + b * a.out_lowp.sb +
                       (int64_t)row * a.out_lowp.st + head * a.out_lowp.sh + d0;
        const __bf16 t0 = (__bf16)val[0], t1 = (__bf16)val[1], t2 = (__bf16)val[2], t3 = (__bf16)val[3];
        const uint32_t p0 =
            (uint32_t)__builtin_bit_cast(uint16_t, t0) | ((uint32_t)__builtin_bit_cast(uint16_t, t1) << 16);
        const uint32_t p1 =
            (uint32_t)__builtin_bit_cast(uint16_t, t2) | ((uint32_t)__builtin_bit_cast(uint16_t, t3) << 16);
        *reinterpret_cast<u32x2*>(lp) = u32x2{p0, p1};
      }
    }
  }
  if (hf == 0) *lse_p = lse_new;
}

// ============================================================================================
// bf16 backward, split into two kernels without any atomics (on this GPU a
// device-wide float atomic is performed past the L2, which caps a fused
// backward's dQ accumulation far below the MFMA rate):
//  * dK/dV kernel: a workgroup owns 128 keys (32 per wave) and walks the query
//    tiles that can see them: S = Q K^T, P, dP = dO V^T, dS, dV^T += dO^T P,
//    dK^T += Q^T dS.  Q/dO tiles are DMA'd one tile ahead.
//  * dQ kernel: a workgroup owns 128 query rows (32 per wave) and walks the
//    key tiles they can see: S^T = K Q^T, P^T, dP^T = V dO^T, dS^T,
//    dQ^T += K^T dS^T.  K/V tiles are DMA'd one tile ahead.
// Both recompute P from the final lse.  With a workspace large enough for
// the bf16 dS of one ring step, the dK/dV kernel also stores dS and dQ = dS K
// is one product (bwd_dq_ds_kernel): five matrix products per pair in all.
// Otherwise the dQ kernel above recomputes S and dP (seven products per pair).
// ============================================================================================

constexpr int DQ_BK = 64;  // keys per dQ-kernel tile

// Blocked dS^T layout of one (batch, head) slice: blocks of 32 keys x 16
// query rows (1 KiB), each stored key-major with the key's 16 rows contiguous;
// blocks ordered by 32-key block, then by 16-row block (ds_ld / 16 of them).
// Element offset of (key, row):
__device__ __forceinline__ int64_t ds_offset(int key, int row, int64_t ds_ld) {
  return ((int64_t)(key >> 5) * (ds_ld >> 4) + (row >> 4)) * 512 + (key & 31) * 16 + (row & 15);
}
// Elements of one slice: keys padded to whole dK/dV key tiles.
__device__ __forceinline__ int64_t ds_slice_elems(int lk, int64_t ds_ld) {
  return (int64_t)((lk + BWD_BK - 1) / BWD_BK * BWD_BK) * ds_ld;
}

// Query tiles (BQB rows) that the dK/dV kernel visits for its key tile kt
// (BWD_BK keys): [q0, q1], empty when q0 > q1.  Both the dK/dV kernel and the
// dQ-from-dS kernel take the range from here, so they agree exactly.
__device__ __forceinline__ void dkdv_query_tiles(const BwdArgs& a, int kt, int& q0, int& q1) {
  const int k_first = kt * BWD_BK;
  const int k_last = min(a.lk, k_first + BWD_BK) - 1;
  const Bounds cf = col_bounds(a.mask, map_pos(a.kmap, k_first));
  const Bounds cl = col_bounds(a.mask, map_pos(a.kmap, k_last));
  const int rbeg = first_ge(a.qmap, cf.lo);
  const int rend = min(a.lq, last_le(a.qmap, cl.hi) + 1);
  q0 = rbeg / BQB;
  q1 = rbeg < rend ? (rend - 1) / BQB : q0 - 1;
}

template <int D>
struct DkdvB {
  static constexpr int NW = 8;                    // waves: 4 key groups x 2 query halves
  static constexpr int TILE = BQB * D * 2;        // one Q (or dO) tile
  static constexpr int OFF_DO = TILE;
  static constexpr int BUF = 2 * TILE;            // a query tile's Q and dO
  static constexpr int NBUF = 2;                  // query tiles are fetched one ahead
  static constexpr int OFF_DEL = BQB * 4;         // lse (natural log, as given), then delta
  static constexpr int LSD = 2 * BQB * 4;
  // The two query buffers come first in LDS (64 KiB for D = 128): every read
  // of them is one per-lane register plus an immediate below 64 KiB, which is
  // what the LDS instruction's offset field holds.  The K and V tiles follow;
  // their read addresses do not change over the loop, and a V address is the
  // matching K address plus an immediate.
  static constexpr int OFF_K = 0;                 // this workgroup's K tile (BWD_BK rows)
  static constexpr int OFF_V = BWD_BK * D * 2;    // and its V tile
};

// dK/dV kernel: 8 waves; wave (kg, qh) owns keys 32*kg.. of the workgroup's
// 128 and query rows 32*qh.. of every 64-row query tile.  K and V rows are
// read from LDS tiles; query tiles (with their lse and delta) are DMA'd one
// tile ahead into two LDS buffers.  Visibility is
// tested per key lane: a query position qp sees this lane's key iff qp lies in
// the key's column interval (col_bounds), so no per-row lookups are needed.
// The two query halves of a key group add their dK/dV through LDS at the end.
template <int D>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_kernel(BwdArgs ap) {
  BwdArgs a = ap;
  int bid = (int)blockIdx.x, nblk = (int)gridDim.x;
  if (ap.g.n) bwd_piece(ap, a, bid, nblk, false);
  using C = DkdvB<D>;
  constexpr int NDB = D / 32;
  // The K/V tiles and the two query-tile buffers are three LDS objects, each
  // buffer reached statically: a read of one buffer then does not wait for
  // the DMA filling the other (the compiler cannot otherwise tell them apart).
  // (the compiler places LDS objects by alignment first: the query buffers'
  // alignment of a whole buffer puts them at the start)
  __shared__ __attribute__((aligned(C::BUF))) char qbuf0[C::BUF];
  __shared__ __attribute__((aligned(C::BUF))) char qbuf1[C::BUF];
  __shared__ __attribute__((aligned(16))) char kv_lds[2 * BWD_BK * D * 2];
  __shared__ __attribute__((aligned(16))) char lsd0[C::LSD];
  __shared__ __attribute__((aligned(16))) char lsd1[C::LSD];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = w & 3, qh = w >> 2;
  const int logical = xcd_logical(bid, nblk);
  const int kt = logical % a.n_ktiles;  // earliest (heaviest causal) key tiles first
  const int bh = logical / a.n_ktiles;
  if (bh >= a.heads * a.batch) return;  // a grouped launch's padding block
  const int head = bh % a.heads, b = bh / a.heads;

  const char* qbase = reinterpret_cast<const char*>(a.q.ptr) + (b * a.q.sb + head * a.q.sh) * 2;
  const char* kbase = reinterpret_cast<const char*>(a.k.ptr) + (b * a.k.sb + head * a.k.sh) * 2;
  const char* vbase = reinterpret_cast<const char*>(a.v.ptr) + (b * a.v.sb + head * a.v.sh) * 2;
  const char* dobase = reinterpret_cast<const char*>(a.dout.ptr) + (b * a.dout.sb + head * a.dout.sh) * 2;
  const Rsrc rq = make_rsrc(qbase, slice_bytes(a.lq, a.q.st, 2, D));
  const Rsrc rk = make_rsrc(kbase, slice_bytes(a.lk, a.k.st, 2, D));
  const Rsrc rv = make_rsrc(vbase, slice_bytes(a.lk, a.v.st, 2, D));
  const Rsrc rdo = make_rsrc(dobase, slice_bytes(a.lq, a.dout.st, 2, D));
  const Rsrc rlse = make_rsrc(a.lse + ((int64_t)b * a.heads + head) * a.lse_sh, (uint32_t)a.lq * 4);
  const Rsrc rdel = make_rsrc(a.delta + ((int64_t)b * a.heads + head) * a.lse_sh, (uint32_t)a.lq * 4);
  const uint32_t qst = (uint32_t)(a.q.st * 2), kst = (uint32_t)(a.k.st * 2);
  const uint32_t vst = (uint32_t)(a.v.st * 2), dst = (uint32_t)(a.dout.st * 2);

  const int k_first = kt * BWD_BK;
  const int k_last = min(a.lk, k_first + BWD_BK) - 1;
  const int kw0 = k_first + 32 * kg;
  const int kw_last = min(k_last, kw0 + 31);
  const bool wave_has_keys = kw0 <= k_last;
  const int key = kw0 + l32;
  const bool key_ok = key <= k_last;
  // Optional dS^T output in the blocked layout of ds_offset(): one wave's
  // 32 keys x 16 rows are one contiguous KiB, so each store instruction writes
  // whole cache lines.  Through a buffer descriptor over this (batch, head)
  // slice, of size 0 when there is no dS^T buffer, so that every store is then
  // dropped (the store itself stays unconditional: a branch around it costs
  // the loop registers).  Every visited (query tile, key) block is written,
  // zeros where nothing is visible, so the dQ kernel reads only written data.
  const bool ds_on = a.dsT != nullptr;
  const int64_t ds_slice = ds_slice_elems(a.lk, a.ds_ld);
  const Rsrc rds = make_rsrc(ds_on ? a.dsT + (int64_t)(b * a.heads + head) * ds_slice : a.dsT,
                             ds_on ? (uint32_t)(ds_slice * 2) : 0u);
  const uint32_t ds_voff = (uint32_t)(ds_offset(l32, 8 * hf, 0) * 2);   // this lane's 16 bytes of a block
  const int ds_kblock = kt * (BWD_BK / 32) + kg;                         // this wave's 32-key block
  const Bounds cb = col_bounds(a.mask, map_pos(a.kmap, min(key, k_last)));       // this lane's key
  const Bounds cbf = col_bounds(a.mask, map_pos(a.kmap, min(kw0, k_last)));      // wave's first key
  const Bounds cbl = col_bounds(a.mask, map_pos(a.kmap, kw_last));               // wave's last key
  // Query positions increase with the row index, so the rows that see this
  // lane's key are one index interval, [ia, ia + ispan] (ia far past every
  // row when none does): a block that is not fully visible is masked with one
  // unsigned compare per score.
  int ia = first_ge(a.qmap, cb.lo), ispan = 0;
  {
    const int ib = min(a.lq - 1, last_le(a.qmap, cb.hi));
    if (ib < ia || !key_ok) ia = 1 << 30;
    else ispan = ib - ia;
  }

  dma_tile<D, BWD_BK, 8>(rk, kst, k_first, kv_lds + C::OFF_K, w, lane);
  dma_tile<D, BWD_BK, 8>(rv, vst, k_first, kv_lds + C::OFF_V, w, lane);
  const char* sK = kv_lds + C::OFF_K;
  const char* sV = kv_lds + C::OFF_V;
  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d) {
    dk[d] = f32x16{};
    dv[d] = f32x16{};
  }

  int qt0, qt1;
  dkdv_query_tiles(a, kt, qt0, qt1);
  const float sl2 = a.scale_log2;

  // Per-lane offsets of the transposed reads within a query tile: rows
  // 32*qh + 8*hf + (j >> 2) + 4*hi at column 32*d + 16*g1 + 4*(j & 3) (j = lane
  // mod 16, g1 = bit 4 of the lane).  The rows 16*u further down sit 16*u*2*D
  // bytes further (the swizzle depends on the row modulo 16 only), so u is an
  // immediate offset rather than another register per read.
  int offT[NDB][2];
  {
    const int j = lane & 15, g1 = (lane >> 4) & 1;
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int colb = 2 * (32 * d + 16 * g1 + 4 * (j & 3));
        offT[d][hi] = nat_off<D>(32 * qh + 8 * hf + (j >> 2) + 4 * hi, colb >> 4) + (colb & 15);
      }
  }
  auto tr_op = [&](const char* tile, int u, int d) {
    const u32x2 lo = tr16(tile + u * 16 * 2 * D + offT[d][0]);
    const u32x2 hi = tr16(tile + u * 16 * 2 * D + offT[d][1]);
    return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
  };

  auto issue = [&](int qtile, char* nb, char* nl) {
    const int r0 = qtile * BQB;
    dma_tile<D, BQB, 8>(rq, qst, r0, nb, w, lane);
    dma_tile<D, BQB, 8>(rdo, dst, r0, nb + C::OFF_DO, w, lane);
    if (w == 0) dma_f32x64(rlse, r0, nl, lane);
    if (w == 1) dma_f32x64(rdel, r0, nl + C::OFF_DEL, lane);
  };

  // dS^T of a tile is stored at the start of the next one: the wait at the end
  // of a tile covers every memory operation of the wave (stores included), and
  // a store issued a whole tile earlier has completed by then.  A wave with
  // nothing pending (no rows in the tile, or before the first tile) stores
  // through a descriptor of size 0, so the stores are dropped (the choice is
  // wave-uniform, so offsets may span the whole 32-bit range of a slice).
  constexpr int kNonTemporal = 2;  // cache-policy bit: dS^T streams out, no reuse before the dQ kernel
  const Rsrc rds_none = make_rsrc(a.dsT, 0u);
  bf16x8 pend[2] = {zero_bf16x8(), zero_bf16x8()};
  bool pend_live = false;
  uint32_t pend_soff = 0;
  auto flush = [&]() {
    const Rsrc rs = pend_live ? rds : rds_none;
#pragma unroll
    for (int u = 0; u < 2; ++u)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, pend[u]), rs, ds_voff, pend_soff + 1024 * u,
                                             kNonTemporal);
  };

  if (qt0 <= qt1) {
    issue(qt0, qbuf0, lsd0);
    wait_vmem();
    __syncthreads();
    // query tile qt from `buf`/`lbuf` while tile qt + 1 is fetched into `nbuf`/`nlbuf`
    auto step = [&](int qt, const char* buf, const char* lbuf, char* nbuf, char* nlbuf) {
      flush();
      const char* sQ = buf;
      const char* sDO = buf + C::OFF_DO;
      const float* sLse = reinterpret_cast<const float*>(lbuf);
      const float* sDel = reinterpret_cast<const float*>(lbuf + C::OFF_DEL);
      // this wave's 32 query rows of the tile
      const int rw0 = qt * BQB + qh * 32;
      const int rwl = min(a.lq - 1, rw0 + 31);
      bool wave_empty = !wave_has_keys || rw0 > rwl;
      bool wave_full = false;
      if (!wave_empty) {
        const int qfirst = map_pos(a.qmap, rw0), qlast = map_pos(a.qmap, rwl);
        wave_empty = qlast < cbf.lo || qfirst > cbl.hi;
        wave_full = (kw0 + 32 <= a.lk) && (rw0 + 32 <= a.lq) && qfirst >= cbl.lo && qlast <= cbf.hi;
      }
      // S = Q K^T and dP = dO V^T, the two chains interleaved with S half of
      // its k-steps ahead, so that S is complete while the last dP products
      // run.
      const int hr0 = qh * 32;
      constexpr int LEAD = D / 32;
      f32x16 s = f32x16{}, dp = f32x16{};
      if (!wave_empty) {
        const int qrow = hr0 + row_perm(l32);
#pragma unroll
        for (int c = 0; c < D / 16 + LEAD; ++c) {
          if (c < D / 16)
            s = mfma_bf16(row_operand<D>(sQ, qrow, c, hf), row_operand<D>(sK, 32 * kg + l32, c, hf), s);
          if (c >= LEAD)
            dp = mfma_bf16(row_operand<D>(sDO, qrow, c - LEAD, hf), row_operand<D>(sV, 32 * kg + l32, c - LEAD, hf),
                           dp);
        }
        // The four operand reads of a k-step are issued one k-step ahead.
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int c = 0; c < D / 16 - 2; ++c) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      }
      // The next query tile is copied in from here, not from the start of the
      // step: its copies then stay out of the S/dP products' operand reads,
      // and half a step is still time enough for them to land.
      if (qt + 1 <= qt1) issue(qt + 1, nbuf, nlbuf);
      if (!wave_empty) {
        // lse (natural log, taken to base 2 in the exponent) and delta of this
        // lane's 16 rows (rows hr0 + 16u + 8hf + i2 for half u) come as two
        // 16-byte reads each.
        f32x4 la[2], lb[2], da[2], db[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int qb = hr0 + 16 * u + 8 * hf;
          la[u] = *reinterpret_cast<const f32x4*>(sLse + qb);
          lb[u] = *reinterpret_cast<const f32x4*>(sLse + qb + 4);
          da[u] = *reinterpret_cast<const f32x4*>(sDel + qb);
          db[u] = *reinterpret_cast<const f32x4*>(sDel + qb + 4);
        }
        // Blocks that are not fully visible set the scores of invisible
        // (query, key) pairs to -inf first, and the lse of a row without any
        // visible key (-inf) to +inf, so that exp2 gives 0 for all of them;
        // what follows is the same straight-line code for every tile.
        if (!wave_full) {
          // row index of score v = rw0 + 8 * hf + 16 * (v >> 3) + (v & 7)
          const int t = rw0 + 8 * hf - ia;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const bool ok = (uint32_t)(t + 16 * (v >> 3) + (v & 7)) <= (uint32_t)ispan;
            s[v] = ok ? s[v] : NEG_INF;
          }
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              la[u][i] = la[u][i] == NEG_INF ? POS_INF : la[u][i];
              lb[u][i] = lb[u][i] == NEG_INF ? POS_INF : lb[u][i];
            }
        }
        // P and dS per half u of this lane's 16 rows, packed to bf16 as they
        // are made.
        bf16x8 pb[2], sb[2];
        auto softmax_row = [&](int u, int i2) {
          const int v = 8 * u + i2;
          const float lse = i2 < 4 ? la[u][i2] : lb[u][i2 - 4];
          const float del = i2 < 4 ? da[u][i2] : db[u][i2 - 4];
          const float e = ex2(__builtin_fmaf(s[v], sl2, -lse * LOG2E));
          pb[u][i2] = (__bf16)e;
          sb[u][i2] = (__bf16)(e * (dp[v] - del));
        };
#pragma unroll
        for (int i2 = 0; i2 < 8; ++i2) softmax_row(0, i2);
        pend[0] = sb[0];
        // The products of half 0, pair by pair, each pair with the operand
        // reads of the next pair and two rows of half 1's softmax; then the
        // products of half 1.  The scheduling fences keep that order.
        bf16x8 op_do = tr_op(sDO, 0, 0), op_q = tr_op(sQ, 0, 0);
#pragma unroll
        for (int k = 0; k < 2 * NDB; ++k) {
          const int u = k / NDB, d = k % NDB;
          bf16x8 nx_do = op_do, nx_q = op_q;
          if (k + 1 < 2 * NDB) {
            nx_do = tr_op(sDO, (k + 1) / NDB, (k + 1) % NDB);
            nx_q = tr_op(sQ, (k + 1) / NDB, (k + 1) % NDB);
          }
          dv[d] = mfma_bf16(op_do, pb[u], dv[d]);
          dk[d] = mfma_bf16(op_q, sb[u], dk[d]);
          if (u == 0) {
#pragma unroll
            for (int i = 0; i < 8 / NDB; ++i) softmax_row(1, (8 / NDB) * d + i);
            if (d == NDB - 1) pend[1] = sb[1];
          }
          __builtin_amdgcn_sched_barrier(0);
          op_do = nx_do;
          op_q = nx_q;
        }
      }
      // This tile's block of dS^T is stored with the next tile; blocks that
      // nothing in them sees are stored as zeros, rows past lq not at all.
      if (wave_empty) {
        pend[0] = zero_bf16x8();
        pend[1] = zero_bf16x8();
      }
      pend_live = rw0 <= rwl;
      pend_soff = (uint32_t)(ds_offset(32 * ds_kblock, rw0, a.ds_ld) * 2);
      wait_vmem();
      __syncthreads();
    };
    for (int qt = qt0; qt <= qt1; qt += 2) {
      step(qt, qbuf0, lsd0, qbuf1, lsd1);
      if (qt + 1 <= qt1) step(qt + 1, qbuf1, lsd1, qbuf0, lsd0);
    }
    flush();
  }
  wait_vmem();  // the K/V tile DMA when no query tile was visited
  __syncthreads();

  // Add the two query halves of each key group: waves qh = 1 park dK^T / dV^T
  // in LDS (reusing the K/V tiles), waves qh = 0 add and write out.
  // Per key group, 4*NDB rows of 64 lanes x 16 bytes: the lanes of one access
  // sit side by side, so a wave's 16-byte writes and reads are conflict free.
  float* red = reinterpret_cast<float*>(kv_lds);  // 4 key groups x 4*NDB x 64 lanes x 4 floats
  constexpr int PER = 16 * NDB;
  float* dkr = reinterpret_cast<float*>(a.dk.ptr) + b * a.dk.sb + (int64_t)key * a.dk.st + head * a.dk.sh;
  float* dvr = reinterpret_cast<float*>(a.dv.ptr) + b * a.dv.sb + (int64_t)key * a.dv.st + head * a.dv.sh;
  float* slot = red + kg * 64 * PER + lane * 4;  // group q = 4d + g at slot + q * 256
  // pass 0: dK (scaled), pass 1: dV
  if (qh == 1) {
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4*>(slot + (4 * d + g) * 256) =
            f32x4{dk[d][4 * g], dk[d][4 * g + 1], dk[d][4 * g + 2], dk[d][4 * g + 3]};
  }
  __syncthreads();
  if (qh == 0 && key_ok) {
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = d * 32 + 8 * g + 4 * hf;
        const f32x4 other = *reinterpret_cast<const f32x4*>(slot + (4 * d + g) * 256);
        f32x4 x = *reinterpret_cast<const f32x4*>(dkr + d0);
        x += a.scale * (f32x4{dk[d][4 * g], dk[d][4 * g + 1], dk[d][4 * g + 2], dk[d][4 * g + 3]} + other);
        *reinterpret_cast<f32x4*>(dkr + d0) = x;
      }
  }
  __syncthreads();
  if (qh == 1) {
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4*>(slot + (4 * d + g) * 256) =
            f32x4{dv[d][4 * g], dv[d][4 * g + 1], dv[d][4 * g + 2], dv[d][4 * g + 3]};
  }
  __syncthreads();
  if (qh == 0 && key_ok) {
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = d * 32 + 8 * g + 4 * hf;
        const f32x4 other = *reinterpret_cast<const f32x4*>(slot + (4 * d + g) * 256);
        f32x4 y = *reinterpret_cast<const f32x4*>(dvr + d0);
        y += f32x4{dv[d][4 * g], dv[d][4 * g + 1], dv[d][4 * g + 2], dv[d][4 * g + 3]} + other;
        *reinterpret_cast<f32x4*>(dvr + d0) = y;
      }
  }
}

template <int D>
struct DqB {
  static constexpr int TILE = DQ_BK * D * 2;
  static constexpr int BUF = 2 * TILE;  // K then V
  static constexpr int LDS = 2 * BUF;
};

template <int D>
__global__ __launch_bounds__(NT, 2) void bwd_dq_kernel(BwdArgs ap) {
  BwdArgs a = ap;
  int bid = (int)blockIdx.x, nblk = (int)gridDim.x;
  if (ap.g.n) bwd_piece(ap, a, bid, nblk, true);
  using C = DqB<D>;
  constexpr int NDB = D / 32;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int logical = xcd_logical(bid, nblk);
  const int qt = a.n_qtiles - 1 - logical % a.n_qtiles;
  const int bh = logical / a.n_qtiles;
  if (bh >= a.heads * a.batch) return;  // a grouped launch's padding block
  const int head = bh % a.heads, b = bh / a.heads;

  const int r_first = qt * FWD_BQ;
  const int r_last = min(a.lq, r_first + FWD_BQ) - 1;
  const int w_first = r_first + 32 * w;
  const int w_last = min(r_last, w_first + 31);
  const bool wave_has_rows = w_first <= r_last;
  const int row = w_first + l32;
  const bool row_ok = row <= r_last;

  const char* qbase = reinterpret_cast<const char*>(a.q.ptr) + (b * a.q.sb + head * a.q.sh) * 2;
  const char* kbase = reinterpret_cast<const char*>(a.k.ptr) + (b * a.k.sb + head * a.k.sh) * 2;
  const char* vbase = reinterpret_cast<const char*>(a.v.ptr) + (b * a.v.sb + head * a.v.sh) * 2;
  const char* dobase = reinterpret_cast<const char*>(a.dout.ptr) + (b * a.dout.sb + head * a.dout.sh) * 2;
  const Rsrc rq = make_rsrc(qbase, slice_bytes(a.lq, a.q.st, 2, D));
  const Rsrc rk = make_rsrc(kbase, slice_bytes(a.lk, a.k.st, 2, D));
  const Rsrc rv = make_rsrc(vbase, slice_bytes(a.lk, a.v.st, 2, D));
  const Rsrc rdo = make_rsrc(dobase, slice_bytes(a.lq, a.dout.st, 2, D));
  const uint32_t qst = (uint32_t)(a.q.st * 2), kst = (uint32_t)(a.k.st * 2);
  const uint32_t vst = (uint32_t)(a.v.st * 2), dst = (uint32_t)(a.dout.st * 2);

  // B operands: Q^T and dO^T columns of this lane's query row.
  bf16x8 qf[D / 16], gf[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    qf[c] = __builtin_bit_cast(bf16x8, bload16(rq, (uint32_t)row * qst + (16 * c + 8 * hf) * 2));
    gf[c] = __builtin_bit_cast(bf16x8, bload16(rdo, (uint32_t)row * dst + (16 * c + 8 * hf) * 2));
  }
  float lse2 = POS_INF, dl = 0.f;
  if (row_ok) {
    const float x = a.lse[((int64_t)b * a.heads + head) * a.lse_sh + row];
    lse2 = (x == NEG_INF) ? POS_INF : x * LOG2E;
    dl = a.delta[((int64_t)b * a.heads + head) * a.lse_sh + row];
  }

  const Bounds rb = row_bounds(a.mask, map_pos(a.qmap, min(row, r_last)));
  const Bounds wg_f = row_bounds(a.mask, map_pos(a.qmap, r_first));
  const Bounds wg_l = row_bounds(a.mask, map_pos(a.qmap, r_last));
  const Bounds wv_f = row_bounds(a.mask, map_pos(a.qmap, min(w_first, r_last)));
  const Bounds wv_l = row_bounds(a.mask, map_pos(a.qmap, w_last));
  const int kbeg = first_ge(a.kmap, wg_f.lo);
  const int kend = min(a.lk, last_le(a.kmap, wg_l.hi) + 1);
  if (kbeg >= kend) return;  // no row of the workgroup sees a key: dQ gains nothing
  const float sl2 = a.scale_log2;
  // The keys this lane's row sees: one index interval [ja, ja + jspan] (key
  // positions increase with the index; ja far past every key when none).
  int ja = first_ge(a.kmap, rb.lo), jspan = 0;
  {
    const int jb = min(a.lk - 1, last_le(a.kmap, rb.hi));
    if (jb < ja || !wave_has_rows) ja = 1 << 30;
    else jspan = jb - ja;
  }

  f32x16 dq[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d) dq[d] = f32x16{};

  if (kbeg < kend) {
    const int jt0 = kbeg / DQ_BK, jt1 = (kend - 1) / DQ_BK;
    dma_tile<D, DQ_BK>(rk, kst, jt0 * DQ_BK, smem, w, lane);
    dma_tile<D, DQ_BK>(rv, vst, jt0 * DQ_BK, smem + C::TILE, w, lane);
    wait_vmem();
    __syncthreads();
    for (int jt = jt0; jt <= jt1; ++jt) {
      const int cur = (jt - jt0) & 1;
      const char* sK = smem + cur * C::BUF;
      const char* sV = sK + C::TILE;
      if (jt < jt1) {
        char* nK = smem + (cur ^ 1) * C::BUF;
        dma_tile<D, DQ_BK>(rk, kst, (jt + 1) * DQ_BK, nK, w, lane);
        dma_tile<D, DQ_BK>(rv, vst, (jt + 1) * DQ_BK, nK + C::TILE, w, lane);
      }
      const int j0 = jt * DQ_BK;
      const int jl = min(a.lk, j0 + DQ_BK) - 1;
      const int kmin = map_pos(a.kmap, j0), kmax = map_pos(a.kmap, jl);
      if (wave_has_rows && kmax >= wv_f.lo && kmin <= wv_l.hi) {
        const bool wave_full = (j0 + DQ_BK <= a.lk) && kmin >= wv_l.lo && kmax <= wv_f.hi;
        const int t = j0 + 8 * hf - ja;  // key index of score (c2, v) = j0 + 8 * hf + 32 * c2 + (v < 8 ? v : v + 8)
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          f32x16 st = f32x16{}, dpt = f32x16{};
          const int krow = c2 * 32 + row_perm(l32);
#pragma unroll
          for (int c = 0; c < D / 16; ++c) st = mfma_bf16(row_operand<D>(sK, krow, c, hf), qf[c], st);
#pragma unroll
          for (int c = 0; c < D / 16; ++c) dpt = mfma_bf16(row_operand<D>(sV, krow, c, hf), gf[c], dpt);
          f32x16 ds;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            float e = ex2(__builtin_fmaf(st[v], sl2, -lse2));
            if (!wave_full) {
              const bool ok = (uint32_t)(t + 32 * c2 + (v < 8 ? v : v + 8)) <= (uint32_t)jspan;
              e = ok ? e : 0.f;
            }
            ds[v] = e * (dpt[v] - dl);
          }
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            bf16x8 sb;
#pragma unroll
            for (int i = 0; i < 8; ++i) sb[i] = (__bf16)ds[8 * u + i];
            const int key0 = c2 * 32 + 16 * u + 8 * hf;
#pragma unroll
            for (int d = 0; d < NDB; ++d) dq[d] = mfma_bf16(tr_operand<D>(sK, key0, d, lane), sb, dq[d]);
          }
        }
      }
      wait_vmem();
      __syncthreads();
    }
  }

  if (!row_ok) return;
  float* dqr = reinterpret_cast<float*>(a.dq.ptr) + b * a.dq.sb + (int64_t)row * a.dq.st + head * a.dq.sh;
#pragma unroll
  for (int d = 0; d < NDB; ++d)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = d * 32 + 8 * g + 4 * hf;
      f32x4 x = *reinterpret_cast<const f32x4*>(dqr + d0);
      x += a.scale * f32x4{dq[d][4 * g], dq[d][4 * g + 1], dq[d][4 * g + 2], dq[d][4 * g + 3]};
      *reinterpret_cast<f32x4*>(dqr + d0) = x;
    }
}

// dQ from the stored dS^T: a workgroup of 8 waves owns 256 query rows (32 per
// wave) and walks the 64-key tiles they can see: dQ^T += K^T dS^T, both
// operands through transposed reads of natural LDS tiles (the K tile, shared
// by all 8 waves, and two dS^T sub-tiles [64 keys][128 rows]).  The kernel
// streams dS^T from HBM, so tiles are DMA'd two ahead through three LDS
// buffers (three separate objects, each reached statically, so the compiler
// waits only for the tile it reads).  A wave skips a key tile whose dK/dV
// workgroup did not visit the wave's query tile: nothing there is visible and
// that block of dS^T was not written.
constexpr int DQS_ROWS = 256;  // query rows per dQ-from-dS workgroup

template <int D>
struct DqsB {
  static constexpr int KT = DQ_BK * D * 2;  // K tile: 64 keys
  static constexpr int ST = DQ_BK * 128 * 2;  // one dS^T sub-tile: 64 keys x 128 query rows
  static constexpr int BUF = KT + 2 * ST;   // one stage
  // buffer->LDS instructions each wave issues per stage (K tile, then the sub-tiles)
  static constexpr int DMA_PER_STAGE = DQ_BK / 8 / (1024 / (2 * D)) + 2 * (DQ_BK / 8 / 4);
};

template <int D>
__global__ __launch_bounds__(512, 1) void bwd_dq_ds_kernel(BwdArgs ap) {
  BwdArgs a = ap;
  int bid = (int)blockIdx.x, nblk = (int)gridDim.x;
  if (ap.g.n) bwd_piece(ap, a, bid, nblk, true);
  using C = DqsB<D>;
  constexpr int NDB = D / 32;
  __shared__ __attribute__((aligned(16))) char sbuf0[C::BUF];
  __shared__ __attribute__((aligned(16))) char sbuf1[C::BUF];
  __shared__ __attribute__((aligned(16))) char sbuf2[C::BUF];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = w >> 2, wcol = w & 3;  // this wave's dS^T sub-tile and its 32-row column block
  const int n_qt = (a.lq + DQS_ROWS - 1) / DQS_ROWS;
  const int logical = xcd_logical(bid, nblk);
  const int qt = n_qt - 1 - logical % n_qt;
  const int bh = logical / n_qt;
  if (bh >= a.heads * a.batch) return;  // a grouped launch's padding block
  const int head = bh % a.heads, b = bh / a.heads;

  const int r_first = qt * DQS_ROWS;
  const int r_last = min(a.lq, r_first + DQS_ROWS) - 1;
  const int w_first = r_first + 32 * w;
  const int row = w_first + l32;
  const bool row_ok = row <= r_last;

  const char* kbase = reinterpret_cast<const char*>(a.k.ptr) + (b * a.k.sb + head * a.k.sh) * 2;
  const Rsrc rk = make_rsrc(kbase, slice_bytes(a.lk, a.k.st, 2, D));
  const uint32_t kst = (uint32_t)(a.k.st * 2);
  // This (batch, head) slice of dS^T (blocked layout, see ds_offset).
  const int64_t ds_elems = ds_slice_elems(a.lk, a.ds_ld);
  const Rsrc rs = make_rsrc(a.dsT + (int64_t)(b * a.heads + head) * ds_elems, (uint32_t)(ds_elems * 2));

  const Bounds wg_f = row_bounds(a.mask, map_pos(a.qmap, r_first));
  const Bounds wg_l = row_bounds(a.mask, map_pos(a.qmap, r_last));
  const int kbeg = first_ge(a.kmap, wg_f.lo);
  const int kend = min(a.lk, last_le(a.kmap, wg_l.hi) + 1);
  if (kbeg >= kend) return;  // no row of the workgroup sees a key: dQ gains nothing
  // The keys this lane's row sees form one index interval [ja, jb] (key
  // positions increase with the index); empty for lanes past the last row.
  // A wave multiplies a tile only when one of its rows sees one of the
  // tile's keys.  The dK/dV kernel has then visited that block of dS^T (a
  // row that sees a key lies in the query range it walks for the key's tile),
  // so only written blocks are used; every other block's dS is zero for
  // these rows.  The test needs no memory access inside the loop.
  int ja = 1 << 30, jb = -1;
  if (row_ok) {
    const Bounds rbd = row_bounds(a.mask, map_pos(a.qmap, row));
    ja = first_ge(a.kmap, rbd.lo);
    jb = min(a.lk - 1, last_le(a.kmap, rbd.hi));
  }

  f32x16 acc[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d) acc[d] = f32x16{};

  // Per-lane byte offsets, within a stage, of the transposed reads of key rows
  // 8*hf + (j >> 2) + 4*hi (j = lane mod 16) at column 32*d + 16*g1 + 4*(j & 3)
  // (g1 = bit 4 of the lane) of the K tile, and at this wave's column block of
  // its dS^T sub-tile.  Key rows 16*ks further sit at an immediate offset (the
  // swizzle depends on the row modulo 16 only).  Keeping every address one
  // register plus an immediate from the stage's buffer also lets the compiler
  // tell the three buffers apart, so reading one does not wait for the DMA
  // into another.
  int offK[NDB][2], offS[2];
  {
    const int j = lane & 15, g1 = (lane >> 4) & 1;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int r = 8 * hf + (j >> 2) + 4 * hi;
#pragma unroll
      for (int d = 0; d < NDB; ++d) {
        const int colb = 2 * (32 * d + 16 * g1 + 4 * (j & 3));
        offK[d][hi] = nat_off<D>(r, colb >> 4) + (colb & 15);
      }
      const int colb = 2 * (32 * wcol + 16 * g1 + 4 * (j & 3));
      offS[hi] = C::KT + half * C::ST + nat_off<128>(r, colb >> 4) + (colb & 15);
    }
  }

  // One stage: the K tile (8 rows per wave), then dS^T keys 8w .. 8w+7 of both
  // sub-tiles into natural swizzled [64][128] tiles: lane l fills LDS position
  // l mod 16 of key 8w + 4i + l/16, which holds the chunk of 8 query rows
  // c = position ^ swz(key).  Each instruction gathers 8 runs of 128 bytes.
  auto issue = [&](int jt, char* buf) {
    dma_tile<D, DQ_BK, 8>(rk, kst, jt * DQ_BK, buf, w, lane);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int kr = 8 * w + 4 * i + (lane >> 4);
        const int c = (lane & 15) ^ swz<128>(kr);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (lds_void*)(buf + C::KT + sub * C::ST + (8 * w + 4 * i) * 256), 16,
            (uint32_t)(ds_offset(jt * DQ_BK + kr, a.ds_row0 + r_first + 128 * sub + 8 * c, a.ds_ld) * 2), 0, 0,
            2 /* non-temporal: dS^T is read once */);
      }
  };

  if (kbeg < kend) {
    const int jt0 = kbeg / DQ_BK, jt1 = (kend - 1) / DQ_BK;
    // Tile jt from `cur` while tile jt + 2 is fetched into `nxt2` (which held
    // tile jt - 1); at the end, wait until tile jt + 1 has landed, leaving tile
    // jt + 2 in flight.  Past the last tile the last one is fetched again into
    // the free buffer, so that every step issues the same copies.
    auto step = [&](int jt, const char* cur, char* nxt2) {
      issue(min(jt + 2, jt1), nxt2);
      if (__any(ja <= jt * DQ_BK + DQ_BK - 1 && jb >= jt * DQ_BK)) {
#pragma unroll
        for (int ks = 0; ks < DQ_BK / 16; ++ks) {
          const u32x2 slo = tr16(cur + offS[0] + ks * 16 * 256), shi = tr16(cur + offS[1] + ks * 16 * 256);
          const bf16x8 sop = __builtin_bit_cast(bf16x8, u32x4{slo[0], slo[1], shi[0], shi[1]});
#pragma unroll
          for (int d = 0; d < NDB; ++d) {
            const u32x2 klo = tr16(cur + offK[d][0] + ks * 16 * 2 * D);
            const u32x2 khi = tr16(cur + offK[d][1] + ks * 16 * 2 * D);
            acc[d] = mfma_bf16(__builtin_bit_cast(bf16x8, u32x4{klo[0], klo[1], khi[0], khi[1]}), sop, acc[d]);
          }
        }
      }
      wait_vmem_keep<C::DMA_PER_STAGE>();
      barrier_keep_vmem();
    };
    issue(jt0, sbuf0);
    issue(min(jt0 + 1, jt1), sbuf1);
    wait_vmem_keep<C::DMA_PER_STAGE>();
    barrier_keep_vmem();
    for (int jt = jt0; jt <= jt1; jt += 3) {
      step(jt, sbuf0, sbuf2);
      if (jt + 1 <= jt1) step(jt + 1, sbuf1, sbuf0);
      if (jt + 2 <= jt1) step(jt + 2, sbuf2, sbuf1);
    }
    // No copy into this workgroup's LDS may still be in flight when its waves end.
    wait_vmem();
  }

  if (!row_ok) return;
  float* dqr = reinterpret_cast<float*>(a.dq.ptr) + b * a.dq.sb + (int64_t)row * a.dq.st + head * a.dq.sh;
#pragma unroll
  for (int d = 0; d < NDB; ++d)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = d * 32 + 8 * g + 4 * hf;
      f32x4 x = *reinterpret_cast<const f32x4*>(dqr + d0);
      x += a.scale * f32x4{acc[d][4 * g], acc[d][4 * g + 1], acc[d][4 * g + 2], acc[d][4 * g + 3]};
      *reinterpret_cast<f32x4*>(dqr + d0) = x;
    }
}

// ============================================================================================
// HBM-bound helpers
// ============================================================================================

// Standalone lse merge: one thread per (row, 4 consecutive d).
__global__ __launch_bounds__(NT) void merge_kernel(MergeArgs a) {
  const int64_t per_row = a.dim / 4;
  const int64_t total = (int64_t)a.batch * a.lq * a.heads * per_row;
  const int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (i >= total) return;
  const int c = (int)(i % per_row);
  int64_t rr = i / per_row;
  const int h = (int)(rr % a.heads);
  rr /= a.heads;
  const int t = (int)(rr % a.lq);
  const int b = (int)(rr / a.lq);
  float* lse_p = a.lse + ((int64_t)b * a.heads + h) * a.lq + t;
  const float la = *lse_p;
  const float lb = a.lse_b[((int64_t)b * a.heads + h) * a.lq + t];
  const float mm = fmaxf(la, lb);
  float wa = 0.f, wb = 0.f;
  if (mm != NEG_INF) {
    const float ea = expf(la - mm), eb = expf(lb - mm);
    const float s = ea + eb;
    wa = ea / s;
    wb = eb / s;
  }
  float* o = reinterpret_cast<float*>(a.out.ptr) + b * a.out.sb + (int64_t)t * a.out.st + h * a.out.sh + 4 * c;
  const float* ob =
      reinterpret_cast<const float*>(a.out_b.ptr) + b * a.out_b.sb + (int64_t)t * a.out_b.st + h * a.out_b.sh + 4 * c;
  const f32x4 x = *reinterpret_cast<const f32x4*>(o);
  const f32x4 y = *reinterpret_cast<const f32x4*>(ob);
  *reinterpret_cast<f32x4*>(o) = wa * x + wb * y;
}

// Second pass of the standalone merge: the lse is rewritten only after every
// output chunk of the row has read the old value (previous launch).

__global__ __launch_bounds__(NT) void merge_lse_kernel(MergeArgs a) {
  const int64_t total = (int64_t)a.batch * a.heads * a.lq;
  const int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (i >= total) return;
  const float la = a.lse[i], lb = a.lse_b[i];
  const float mm = fmaxf(la, lb);
  a.lse[i] = (mm == NEG_INF) ? NEG_INF : mm + logf(expf(la - mm) + expf(lb - mm));
}

// delta[b, h, t] = sum_d dout * out.  16 lanes per row.
template <bool BF16>
__global__ __launch_bounds__(NT) void prep_kernel(PrepArgs a) {
  const int64_t rows = (int64_t)a.batch * a.lq * a.heads;
  const int64_t rid = (int64_t)blockIdx.x * (NT / 16) + threadIdx.x / 16;
  const int sub = threadIdx.x & 15;
  float acc = 0.f;
  int b = 0, t = 0, h = 0;
  if (rid < rows) {
    h = (int)(rid % a.heads);
    int64_t rr = rid / a.heads;
    t = (int)(rr % a.lq);
    b = (int)(rr / a.lq);
    const float* o = reinterpret_cast<const float*>(a.out.ptr) + b * a.out.sb + (int64_t)t * a.out.st + h * a.out.sh;
    for (int d = sub * 4; d < a.dim; d += 64) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(o + d);
      float y0, y1, y2, y3;
      if constexpr (BF16) {
        const uint16_t* g = reinterpret_cast<const uint16_t*>(a.dout.ptr) + b * a.dout.sb + (int64_t)t * a.dout.st +
                            h * a.dout.sh + d;
        const u32x2 u = *reinterpret_cast<const u32x2*>(g);
        y0 = __uint_as_float(u[0] << 16);
        y1 = __uint_as_float(u[0] & 0xffff0000u);
        y2 = __uint_as_float(u[1] << 16);
        y3 = __uint_as_float(u[1] & 0xffff0000u);
      } else {
        const f32x4 y = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(a.dout.ptr) + b * a.dout.sb +
                                                        (int64_t)t * a.dout.st + h * a.dout.sh + d);
        y0 = y[0]; y1 = y[1]; y2 = y[2]; y3 = y[3];
      }
      acc += x[0] * y0 + x[1] * y1 + x[2] * y2 + x[3] * y3;
    }
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 16);
  if (rid < rows && sub == 0) a.delta[((int64_t)b * a.heads + h) * a.lq + t] = acc;
}

__global__ __launch_bounds__(NT) void zero_kernel(Tensor4W t, int32_t batch, int32_t heads, int32_t rows, int32_t dim) {
  const int64_t per_row = dim / 4;
  const int64_t total = (int64_t)batch * rows * heads * per_row;
  const int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (i >= total) return;
  const int c = (int)(i % per_row);
  int64_t rr = i / per_row;
  const int h = (int)(rr % heads);
  rr /= heads;
  const int r = (int)(rr % rows);
  const int b = (int)(rr / rows);
  float* o = reinterpret_cast<float*>(t.ptr) + b * t.sb + (int64_t)r * t.st + h * t.sh + 4 * c;
  *reinterpret_cast<f32x4*>(o) = f32x4{0.f, 0.f, 0.f, 0.f};
}

// fp32 -> bf16, round to nearest, ties to even, on the bit pattern (so the
// result does not depend on the wave's float mode: subnormals round like any
// other value); a NaN stays a NaN with its sign and top payload bits, quieted.
__device__ __forceinline__ uint32_t bf16_bits_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x0040u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Eight elements per thread: two 16-byte loads and one 16-byte store when
// both pointers are 16-byte aligned, element by element otherwise (and in the
// last, partial group).
__global__ __launch_bounds__(NT) void cast_kernel(const float* src, uint16_t* dst, int64_t n, int vec) {
  const int64_t i = ((int64_t)blockIdx.x * NT + threadIdx.x) * 8;
  if (i >= n) return;
  if (vec && i + 8 <= n) {
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(src + i);
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(src + i + 4);
    u32x4 w;
    w[0] = bf16_bits_rne(x0[0]) | (bf16_bits_rne(x0[1]) << 16);
    w[1] = bf16_bits_rne(x0[2]) | (bf16_bits_rne(x0[3]) << 16);
    w[2] = bf16_bits_rne(x1[0]) | (bf16_bits_rne(x1[1]) << 16);
    w[3] = bf16_bits_rne(x1[2]) | (bf16_bits_rne(x1[3]) << 16);
    *reinterpret_cast<u32x4*>(dst + i) = w;
    return;
  }
  const int64_t e = i + 8 < n ? i + 8 : n;
  for (int64_t j = i; j < e; ++j) dst[j] = (uint16_t)bf16_bits_rne(src[j]);
}

inline unsigned blocks_for(int64_t n) { return (unsigned)((n + NT - 1) / NT); }

}  // namespace

// ============================================================================================
// Fixed scratch of ra_ring_bwd_noalloc (callers that cannot allocate): one
// array per GPU, held until the process ends.  Host code reaches it only
// through the address hipGetSymbolAddress returns for the current device.
// ============================================================================================

constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

size_t scratch_capacity() { return kScratchBytes; }

hipError_t scratch_device_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// ============================================================================================
// Launchers
// ============================================================================================

// Grid of a grouped launch: each piece gets ceil(n / rows) x heads x batch
// blocks, rounded up to a multiple of 8, where n is the piece's length, or
// for the query-side kernels (`qside`) its rows from qoff on; fills g.wg_begin.
static unsigned group_grid(PieceTable& g, int rows, int heads, int batch, bool qside) {
  int64_t acc = 0;
  for (int p = 0; p < g.n; ++p) {
    g.wg_begin[p] = (int32_t)acc;
    const int64_t n = g.len[p] - (qside ? g.qoff[p] : 0);
    const int64_t blocks = (int64_t)((n + rows - 1) / rows) * heads * batch;
    acc += (blocks + 7) / 8 * 8;
  }
  g.wg_begin[g.n] = (int32_t)acc;
  return (unsigned)acc;
}

hipError_t launch_fwd(const FwdArgs& a0, int head_dim, bool bf16, hipStream_t s) {
  FwdArgs a = a0;
  const unsigned grid = a.g.n ? group_grid(a.g, FWD_BQ, a.heads, a.batch, true)
                              : (unsigned)((int64_t)a.n_qtiles * a.heads * a.batch);
  if (grid == 0) return hipSuccess;
  if (a.g.n && !bf16) return hipErrorInvalidValue;  // only the bf16 kernel takes a piece table
  if (bf16) {
    if (head_dim == 128) hipLaunchKernelGGL((fwd_kernel_bf16<128>), dim3(grid), dim3(NT), 0, s, a);
    else hipLaunchKernelGGL((fwd_kernel_bf16<64>), dim3(grid), dim3(NT), 0, s, a);
  } else {
    if (head_dim == 128) hipLaunchKernelGGL((fwd_kernel<128, false>), dim3(grid), dim3(NT), 0, s, a);
    else hipLaunchKernelGGL((fwd_kernel<64, false>), dim3(grid), dim3(NT), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_fused_f32(const BwdArgs& a, int head_dim, hipStream_t s) {
  const unsigned grid = (unsigned)((int64_t)a.n_ktiles * a.heads * a.batch);
  if (grid == 0) return hipSuccess;
  if (head_dim == 128) hipLaunchKernelGGL((bwd_kernel<128, false>), dim3(grid), dim3(NT), 0, s, a);
  else hipLaunchKernelGGL((bwd_kernel<64, false>), dim3(grid), dim3(NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const BwdArgs& a0, int head_dim, hipStream_t s) {
  BwdArgs a = a0;
  const unsigned grid = a.g.n ? group_grid(a.g, BWD_BK, a.heads, a.batch, false)
                              : (unsigned)((int64_t)a.n_ktiles * a.heads * a.batch);
  if (grid == 0) return hipSuccess;
  if (head_dim == 128) hipLaunchKernelGGL((bwd_dkdv_kernel<128>), dim3(grid), dim3(512), 0, s, a);
  else hipLaunchKernelGGL((bwd_dkdv_kernel<64>), dim3(grid), dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dq_ds(const BwdArgs& a0, int head_dim, hipStream_t s) {
  BwdArgs a = a0;
  const unsigned grid = a.g.n ? group_grid(a.g, DQS_ROWS, a.heads, a.batch, true)
                              : (unsigned)((int64_t)((a.lq + DQS_ROWS - 1) / DQS_ROWS) * a.heads * a.batch);
  if (grid == 0) return hipSuccess;
  if (head_dim == 128) hipLaunchKernelGGL((bwd_dq_ds_kernel<128>), dim3(grid), dim3(512), 0, s, a);
  else hipLaunchKernelGGL((bwd_dq_ds_kernel<64>), dim3(grid), dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdArgs& a0, int head_dim, hipStream_t s) {
  BwdArgs a = a0;
  const unsigned grid = a.g.n ? group_grid(a.g, FWD_BQ, a.heads, a.batch, true)
                              : (unsigned)((int64_t)a.n_qtiles * a.heads * a.batch);
  if (grid == 0) return hipSuccess;
  if (head_dim == 128) hipLaunchKernelGGL((bwd_dq_kernel<128>), dim3(grid), dim3(NT), 0, s, a);
  else hipLaunchKernelGGL((bwd_dq_kernel<64>), dim3(grid), dim3(NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  const int64_t n_out = (int64_t)a.batch * a.lq * a.heads * (a.dim / 4);
  const int64_t n_lse = (int64_t)a.batch * a.heads * a.lq;
  if (n_out == 0) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel, dim3(blocks_for(n_out)), dim3(NT), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(merge_lse_kernel, dim3(blocks_for(n_lse)), dim3(NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_prep(const PrepArgs& a, bool bf16, hipStream_t s) {
  const int64_t rows = (int64_t)a.batch * a.lq * a.heads;
  if (rows == 0) return hipSuccess;
  const unsigned grid = (unsigned)((rows + NT / 16 - 1) / (NT / 16));
  if (bf16) hipLaunchKernelGGL(prep_kernel<true>, dim3(grid), dim3(NT), 0, s, a);
  else hipLaunchKernelGGL(prep_kernel<false>, dim3(grid), dim3(NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_cast(const float* src, void* dst, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int vec = (((uintptr_t)src | (uintptr_t)dst) & 15) == 0 ? 1 : 0;
  hipLaunchKernelGGL(cast_kernel, dim3(blocks_for((n + 7) / 8)), dim3(NT), 0, s, src,
                     reinterpret_cast<uint16_t*>(dst), n, vec);
  return hipGetLastError();
}

hipError_t launch_zero(const Tensor4W& t, int32_t batch, int32_t heads, int32_t rows, int32_t dim, hipStream_t s) {
  const int64_t n = (int64_t)batch * rows * heads * (dim / 4);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_kernel, dim3(blocks_for(n)), dim3(NT), 0, s, t, batch, heads, rows, dim);
  return hipGetLastError();
}

}  // namespace ra
