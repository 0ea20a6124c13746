// Internal interface between the host planner (ra_host.cpp) and the gfx950
// kernels (ra_kernels.hip).  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

// Posmap as the kernels see it: int32 positions (seq_len < 2^31 is validated).
struct DSeg {
  int32_t begin, stride, len;
};
struct DMap {
  int32_t nseg;
  DSeg s0, s1;
  int32_t total;  // s0.len + (nseg == 2 ? s1.len : 0)
};

// Per-row visibility: key position kp is visible to query position qp iff
// lo(qp) <= kp <= hi(qp), with lo/hi from the causal flag and cu_seqlens.
struct MaskSpec {
  int32_t causal;
  int32_t nseq;       // 0: one sequence
  const int32_t* cu;  // device cu_seqlens [nseq+1]
};

struct Tensor4 {
  const void* ptr;
  int64_t sb, st, sh;  // element strides
};
struct Tensor4W {
  void* ptr;
  int64_t sb, st, sh;
};

enum FwdMode : int32_t { FWD_STORE = 0, FWD_MERGE = 1 };

// Independent rings in one launch (the sequences of a per-sequence layout, all
// at the same ring step).  Piece p is rows [row0[p], row0[p] + len[p]) of the
// q/out/lse (and of every k/v block and gradient) buffers, with its own
// posmaps; its workgroups are blocks [wg_begin[p], wg_begin[p+1]) of the grid,
// a multiple of 8 per piece so that the XCD mapping holds within each piece
// (blocks past the piece's own count return at once).  wg_begin is filled by
// the launch function of each kernel (block counts differ per kernel).
constexpr int kMaxPieces = 16;
struct PieceTable {
  int32_t n;  // 0: not a grouped launch
  int32_t wg_begin[kMaxPieces + 1];
  int32_t row0[kMaxPieces], len[kMaxPieces];
  int32_t flags[kMaxPieces];  // forward: bit 0 merge into out/lse (else store), bit 1 write out_lowp
  // Forward and dQ kernels: the first query row (within the piece, a multiple
  // of 16) of the rows they process; the rows before it see no key at this
  // step.  The dK/dV kernel always takes all of the piece's query rows.
  int32_t qoff[kMaxPieces];
  DMap qmap[kMaxPieces], kmap[kMaxPieces];
  int64_t ds_off[kMaxPieces];  // backward: element offset of the piece's dS^T region
  int64_t ds_ld[kMaxPieces];
};
constexpr int32_t PIECE_MERGE = 1, PIECE_LOWP = 2;

struct FwdArgs {
  Tensor4 q, k, v;
  Tensor4W out;      // fp32
  float* lse;        // fp32, row t of (batch b, head h) at lse[(b*heads + h)*lse_sh + t]
  int64_t lse_sh;    // head stride of lse (lq unless the rows are a slice of a longer buffer)
  Tensor4W out_lowp; // optional, ptr may be null; same dtype as q
  int32_t batch, heads, lq, lk;
  DMap qmap, kmap;
  MaskSpec mask;
  float scale_log2;  // softmax_scale * log2(e)
  int32_t mode;      // FwdMode
  int32_t n_qtiles;
  PieceTable g;      // grouped launch (bf16 kernel only), g.n = 0 otherwise
};

struct BwdArgs {
  Tensor4 q, k, v, dout;
  const float* lse;    // natural log (final); row t of (b, h) at lse[(b*heads + h)*lse_sh + t]
  const float* delta;  // same indexing as lse
  int64_t lse_sh;      // head stride of lse and delta (lq unless the rows are a slice)
  Tensor4W dq, dk, dv; // fp32 accumulators
  int32_t batch, heads, lq, lk;
  DMap qmap, kmap;
  MaskSpec mask;
  float scale;         // softmax_scale
  float scale_log2;    // softmax_scale * log2(e)
  int32_t n_ktiles;    // key tiles (dK/dV and fused kernels)
  int32_t n_qtiles;    // query tiles (dQ kernels)
  // bf16 dS^T [b][h][lk][ds_ld] (query rows contiguous), or null.  Written by
  // the dK/dV kernel when set; read by the dQ-from-dS kernel.
  uint16_t* dsT;
  int64_t ds_ld;
  int32_t ds_row0;   // dQ-from-dS: dS^T row of this launch's query row 0 (a multiple of 16)
  PieceTable g;      // grouped launch (bf16 kernels only), g.n = 0 otherwise
};

struct MergeArgs {
  Tensor4W out;
  float* lse;
  Tensor4 out_b;  // fp32
  const float* lse_b;
  int32_t batch, heads, lq, dim;
};

struct PrepArgs {
  Tensor4 out;   // fp32
  Tensor4 dout;  // dtype
  float* delta;  // [b, h, lq]
  int32_t batch, heads, lq, dim;
};

// Kernel ids reported by the timing facility.
enum KernelId : int32_t {
  K_FWD = 0,
  K_BWD = 1,  // bf16: dK/dV kernel; fp32: fused backward
  K_MERGE = 2,
  K_PREP = 3,
  K_CAST = 5,
  K_ZERO = 6,
  K_BWD_DQ = 7,     // bf16 dQ kernel (recomputes S and dP)
  K_BWD_DQ_DS = 8,  // bf16 dQ kernel reading the stored dS
  K_COUNT = 9
};

// Tile sizes shared by planner and kernels.
constexpr int FWD_BQ = 128;  // query rows per forward workgroup
constexpr int BWD_BK = 128;  // key rows per backward workgroup

// Launchers (ra_kernels.hip).  Return the launch status; the caller checks it.
hipError_t launch_fwd(const FwdArgs& a, int head_dim, bool bf16, hipStream_t s);
hipError_t launch_bwd_fused_f32(const BwdArgs& a, int head_dim, hipStream_t s);
hipError_t launch_bwd_dkdv(const BwdArgs& a, int head_dim, hipStream_t s);
hipError_t launch_bwd_dq(const BwdArgs& a, int head_dim, hipStream_t s);
hipError_t launch_bwd_dq_ds(const BwdArgs& a, int head_dim, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, hipStream_t s);
hipError_t launch_prep(const PrepArgs& a, bool bf16, hipStream_t s);
hipError_t launch_cast(const float* src, void* dst, int64_t n, hipStream_t s);
// Fixed device scratch of the no-allocation entry point (ra_kernels.hip): its
// size, and its address on the current device (looked up once per device with
// hipGetSymbolAddress; the array's host-side name is not a device address).
size_t scratch_capacity();
hipError_t scratch_device_ptr(void** out);
hipError_t launch_zero(const Tensor4W& t, int32_t batch, int32_t heads, int32_t rows, int32_t dim,
                       hipStream_t s);

}  // namespace ra
