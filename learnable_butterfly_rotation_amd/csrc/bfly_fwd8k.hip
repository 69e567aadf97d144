// The butterfly of length 8192 (13 stages), in two passes.  Its stages
// 0..11 pair elements within each half (bit 12 fixed), so they are two
// independent butterflies of length 4096 whose angles are the halves of
// each stage's angle row; stage 12 pairs element i with i + 4096 (ButterflyQuant
// abstract: log2 n stages of Givens rotations; the duidaima.com write-up,
// section "butterfly": the recursive structure for powers of two).  The
// 13-stage coefficient set does not fit in one thread's registers beside
// its rows, so:
//   pass 1: the fused forward kernel of length 4096 on both halves in one
//           launch (grid y = the half; rows 8192 elements apart, each half
//           with its own table), fp32 out into the caller's workspace;
//   pass 2: final_stage_kernel applies stage 12 to the two halves column by
//           column and stores y (bf16 or fp32) and the group codes, with the
//           fused kernel's quantizer.
// The table of n = 8192: the two half tables (layout of n = 4096), then
// (cos, sin) of stage 12's 4096 angles.
#include <string.h>

#include "bfly_fwd_kernel.h"

namespace bfly {
namespace {

constexpr int H8K = 4096, N8K = 8192;
constexpr int FS_THREADS = H8K / 8;  // 8 columns of each half per thread: one row per pass

struct FinalParams {
  const float* v;    // [rows][8192] fp32: both halves after their 12 stages
  const float2* cs;  // [4096] (cos, sin) of stage 12's angles
  void* y;           // [rows][8192] bf16 or fp32, or nullptr
  uint8_t* codes;    // nullptr: no quantization
  uint16_t* scales;
  uint16_t* zeros;
  int64_t rows;
  int32_t bits, group, asym;
};

// One row per workgroup pass (grid-stride over rows).  Thread t holds
// columns 8t..8t+7 of both halves, so a quantization group (group/8
// consecutive lanes, group <= 512) lies in one wave, as in the fused kernel.
template <int YK>
__global__ void __launch_bounds__(FS_THREADS) final_stage_kernel(FinalParams P) {
  const int t = threadIdx.x;
  const int c0 = 8 * t;
  float cc[8], sn[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float4 q = reinterpret_cast<const float4*>(P.cs + c0)[k];
    cc[2 * k] = q.x;
    sn[2 * k] = q.y;
    cc[2 * k + 1] = q.z;
    sn[2 * k + 1] = q.w;
  }
  const bool quant = P.codes != nullptr;
  const int bits = P.bits;
  const bool asym = P.asym != 0;
  const int gt = quant ? P.group / 8 : 1;
  const float top = asym ? (float)((1 << bits) - 1) : (float)((1 << (bits - 1)) - 1);
  const float inv_top = 1.0f / top;
  const int ngr = quant ? N8K / P.group : 0;
  const bool scale_lane = quant && (t & (gt - 1)) == 0;
  // Per row, buffer resources covering exactly that row of each array; a
  // lane with no scale to store aims outside its range.  The next row's
  // input is loaded before this row's arithmetic and stores (a row past the
  // end has an empty range: its loads return zeros and move no data).
  const int64_t G = gridDim.x;
  uint4 in[2][2];
  auto load_row = [&](const int64_t r) {
    const auto rv = buffer_range32(P.v + (r < P.rows ? r : 0) * N8K, r < P.rows ? N8K * 4 : 0);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      in[0][k] = buf_ld16<kNonTemporal>(rv, (uint32_t)(c0 + 4 * k) * 4);
      in[1][k] = buf_ld16<kNonTemporal>(rv, (uint32_t)(H8K + c0 + 4 * k) * 4);
    }
  };
  load_row(blockIdx.x);
  for (int64_t r = blockIdx.x; r < P.rows; r += G) {
    float lo[8], hi[8];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint4 a = in[0][k], b = in[1][k];
      lo[4 * k] = __uint_as_float(a.x); lo[4 * k + 1] = __uint_as_float(a.y);
      lo[4 * k + 2] = __uint_as_float(a.z); lo[4 * k + 3] = __uint_as_float(a.w);
      hi[4 * k] = __uint_as_float(b.x); hi[4 * k + 1] = __uint_as_float(b.y);
      hi[4 * k + 2] = __uint_as_float(b.z); hi[4 * k + 3] = __uint_as_float(b.w);
    }
    load_row(r + G);
    float w[2][8];  // stage 12: (v_i, v_j) -> (c v_i - s v_j, s v_i + c v_j)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      w[0][e] = fmaf(cc[e], lo[e], -(sn[e] * hi[e]));
      w[1][e] = fmaf(sn[e], lo[e], cc[e] * hi[e]);
    }
    const auto ry = buffer_range32(static_cast<uint16_t*>(P.y) + (YK == Y_BF16 ? r * N8K : 0),
                                   YK == Y_BF16 ? N8K * 2 : 0);
    const auto ry4 = buffer_range32(static_cast<float*>(P.y) + (YK == Y_F32 ? r * N8K : 0),
                                    YK == Y_F32 ? N8K * 4 : 0);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t col = (uint32_t)(h * H8K + c0);  // within the row
      if (YK == Y_BF16) {
        buf_st16<kNonTemporal>(ry, col * 2,
                               make_uint4(pack_bf16(w[h][0], w[h][1]), pack_bf16(w[h][2], w[h][3]),
                                          pack_bf16(w[h][4], w[h][5]), pack_bf16(w[h][6], w[h][7])));
      } else if (YK == Y_F32) {
#pragma unroll
        for (int k = 0; k < 2; ++k)
          buf_st16<kNonTemporal>(ry4, (col + 4 * k) * 4,
                                 make_uint4(__float_as_uint(w[h][4 * k]), __float_as_uint(w[h][4 * k + 1]),
                                            __float_as_uint(w[h][4 * k + 2]),
                                            __float_as_uint(w[h][4 * k + 3])));
      }
      if (quant) {  // uniform across the workgroup
        const QParams q = quant_params(w[h], gt, asym, inv_top, top);
        quant_clamp(w[h], q);
        const uint32_t packed = quant_pack(w[h], q, bits, asym);
        const auto rc = buffer_range32(P.codes + r * (N8K * bits / 8), (uint32_t)(N8K * bits / 8));
        if (bits == 4) buf_st4<kNonTemporal>(rc, col / 2, packed);
        else buf_st2<kNonTemporal>(rc, col / 4, (uint16_t)packed);
        const auto rs = buffer_range32(P.scales + r * ngr, (uint32_t)ngr * 2);
        const uint32_t off = scale_lane ? 2 * (col / P.group) : kOutOfRange;
        buf_st2<kNonTemporal>(rs, off, (uint16_t)(q.sz & 0xFFFFu));
        if (asym) {
          const auto rz = buffer_range32(P.zeros + r * ngr, (uint32_t)ngr * 2);
          buf_st2<kNonTemporal>(rz, off, (uint16_t)(q.sz >> 16));
        }
      }
    }
  }
}

template <int YK>
hipError_t launch_final(const FinalParams& p, hipStream_t s) {
  auto kern = final_stage_kernel<YK>;
  int per_cu = 0, num_cu = 0;
  const hipError_t e =
      kernel_setup(reinterpret_cast<const void*>(kern), FS_THREADS, 0, &per_cu, &num_cu);
  if (e != hipSuccess) return e;
  const int64_t cap = (int64_t)per_cu * num_cu;
  const int grid = (int)(p.rows < cap ? p.rows : cap);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(FS_THREADS), 0, s, p);
  return hipGetLastError();
}

}  // namespace

size_t table8k_bytes() { return 2 * table_bytes(12) + (size_t)H8K * sizeof(float2); }

hipError_t launch_forward_8192(const Fwd8kParams& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  const char* base = static_cast<const char*>(a.table);
  {
    // both halves in one launch (grid y = the half; the kernel offsets the
    // columns and the table of the upper half)
    FwdParams p;
    memset(&p, 0, sizeof(p));
    p.x = a.x;
    p.y = a.v;
    p.rows = a.rows;
    p.m = 1;
    p.lognb = 12;
    p.x_bf16 = a.x_bf16;
    p.y_kind = Y_F32;
    p.tab = table_at(base, 12);
    const hipError_t e = a.x_bf16 ? launch_fwd_variant<12, 1, 2, true, Y_F32, Q_NONE, 2>(p, s)
                                  : launch_fwd_variant<12, 1, 2, false, Y_F32, Q_NONE, 2>(p, s);
    if (e != hipSuccess) return e;
  }
  FinalParams f;
  f.v = a.v;
  f.cs = reinterpret_cast<const float2*>(base + 2 * table_bytes(12));
  f.y = a.y;
  f.codes = a.codes;
  f.scales = a.scales;
  f.zeros = a.zeros;
  f.rows = a.rows;
  f.bits = a.bits;
  f.group = a.group;
  f.asym = a.asym;
  if (a.y_kind == Y_BF16) return launch_final<Y_BF16>(f, s);
  if (a.y_kind == Y_F32) return launch_final<Y_F32>(f, s);
  return launch_final<Y_NONE>(f, s);
}

}  // namespace bfly
