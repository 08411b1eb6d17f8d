// gdn_linear.hip -- token-parallel linear layers around the mixer, on bf16 MFMA.
//
// The mixer's inputs are projections of the hidden states and its output is
// projected back ("Qwen3.8-Flash-Next" tech report, Fig. 2 caption: the projected
// query, key and value streams; "Qwen3-Next 80B-A3B" field guide, cutaway 02: the
// gated output is projected).  Both are plain GEMMs C = A W^T with A [M, K] (tokens x
// features) and W [N, K] (one row of weights per output feature), bf16 operands and
// fp32 accumulation.  The epilogue scatters column ranges of C into separate output
// tensors, so the in-projection writes q, k, v, z (bf16) and a, b (fp32) in exactly
// the layouts the mixer reads, with no intermediate buffer.
//
// Tiling: one workgroup of 8 waves computes a 256 x 256 block of C, K in steps of
// 64 through double-buffered LDS tiles (one barrier per step): the next step's tiles
// go from global memory straight into the other LDS buffer (buffer loads with the LDS
// destination, no register staging) while the current one is multiplied.  Wave (wm, wn) owns
// rows 64 wm .. + 63 and columns 128 wn .. + 127: 2 x 4 products
// v_mfma_f32_32x32x16_bf16 per 16-wide k slice (128 accumulators per lane).
#include "gdn_device.h"
#include "gdn_linear.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 256, kBN = 256, kBK = 64;
// waves along M and N; a wave computes a kWaveRows x kWaveCols block of C from
// MT x NT 32 x 32 MFMA tiles
constexpr int kWavesM = 4, kWavesN = 2;
constexpr int kLinWaves = kWavesM * kWavesN, kLinThreads = 64 * kLinWaves;
constexpr int kWaveRows = kBM / kWavesM, kWaveCols = kBN / kWavesN;
constexpr int MT = kWaveRows / 32, NT = kWaveCols / 32;
constexpr int kLoadsPerWave = 32 / kLinWaves;  // 1 KB blocks of each 32 KB tile
// LDS tiles [256 rows][64 k] bf16, unpadded (128-byte rows), filled straight from global
// memory: a wave's 16-byte load writes 64 consecutive 16-byte slots (8 rows).  The k
// chunk g (8 bf16) of row r sits in slot g ^ (r & 7) ^ ((r >> 3) & 1) of its row, so the
// 16-byte operand reads of 16 consecutive rows at one g hit distinct banks.
constexpr int kTileBytes = kBM * kBK * 2;                  // 32 KB
constexpr size_t kLinLds = 2 * 2 * (size_t)kTileBytes;   // A and B, 2 buffers: 128 KB
static_assert(kLinLds <= 160 * 1024, "LDS budget");

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ int swz_slot(int row, int g) { return g ^ (row & 7) ^ ((row >> 3) & 1); }

// kTileSeg: every segment boundary is a multiple of 32, so each 32-column MFMA tile lies in
// one segment (a scalar lookup) and its stores are raw buffer stores: a per-lane column
// offset, a scalar row offset, and the buffer's bound dropping rows past M.
template <bool kTileSeg>
__global__ void __launch_bounds__(kLinThreads, 1)
linear_bf16_kernel(const bf16_t *__restrict__ A, const bf16_t *__restrict__ W, int64_t M, int N,
                   int K, LinearOut out) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % kWavesM, wn = wave / kWavesM;
  // column blocks fastest: consecutive workgroups share their rows of A (in L2)
  const int nblk = (N + kBN - 1) / kBN;
  const int64_t m0 = (int64_t)(blockIdx.x / nblk) * kBM;
  const int n0 = (int)(blockIdx.x % nblk) * kBN;

  // one buffer per operand over this block's rows: rows past M or N read as zero
  const int64_t rowsA = M - m0 < kBM ? M - m0 : kBM;
  const int rowsB = N - n0 < kBN ? N - n0 : kBN;
  const __amdgpu_buffer_rsrc_t ra = rsrc(A + m0 * K, (uint32_t)(rowsA * K * 2));
  const __amdgpu_buffer_rsrc_t rb = rsrc(W + (int64_t)n0 * K, (uint32_t)((int64_t)rowsB * K * 2));

  // loads of one K step: wave w fills 8-row blocks kLoadsPerWave w .. of each tile; lane l
  // takes row 8b + l/8 and slot l%8, i.e. the global chunk swz_slot(row, l%8) of that row
  uint32_t voff[kLoadsPerWave];
#pragma unroll
  for (int i = 0; i < kLoadsPerWave; ++i) {
    const int row = 8 * (kLoadsPerWave * wave + i) + (lane >> 3);
    voff[i] = (uint32_t)(row * K * 2 + swz_slot(row, lane & 7) * 16);
  }
  typedef __attribute__((address_space(3))) void lds_void;
  auto gload = [&](int k0, int buf) {
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i) {
      const int blk = (buf * 2 * kTileBytes) + (kLoadsPerWave * wave + i) * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(smem + blk), 16, voff[i], k0 * 2, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)(smem + blk + kTileBytes), 16, voff[i],
                                               k0 * 2, 0, 0);
    }
  };

  f32x16 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mt][nt][r] = 0.f;

  const int nk = K / kBK;
  gload(0, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's tile loads are in LDS
  __syncthreads();
  // operand rows of this lane: A rows kWaveRows wm + 32 mt + (lane % 32), W rows
  // kWaveCols wn + 32 nt + (lane % 32); k chunk 2 kk + lane / 32 of the step
  const int lr = lane & 31, kh = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * kBK, buf ^ 1);  // the other buffer was last read before the barrier
    const unsigned char *tA = smem + buf * 2 * kTileBytes;
    const unsigned char *tB = tA + kTileBytes;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int g = 2 * kk + kh;
      bf16x8_t af[MT], bfr[NT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int row = kWaveRows * wm + 32 * mt + lr;
        af[mt] = *reinterpret_cast<const bf16x8_t *>(tA + row * 128 + swz_slot(row, g) * 16);
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int row = kWaveCols * wn + 32 * nt + lr;
        bfr[nt] = *reinterpret_cast<const bf16x8_t *>(tB + row * 128 + swz_slot(row, g) * 16);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mt], bfr[nt], acc[mt][nt], 0,
                                                                 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the next step's tiles are in LDS
    __syncthreads();
  }

  // epilogue: lane holds column (lane % 32) and rows 8 (r / 4) + 4 (lane / 32) + (r % 4) of
  // each 32 x 32 tile
  if constexpr (kTileSeg) {
    const int64_t r0 = m0 + kWaveRows * wm;  // this wave's first row
    const int64_t rows = M - r0 < kWaveRows ? M - r0 : kWaveRows;
    const int ln = lane & 31, lh = lane >> 5;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int nbase = n0 + kWaveCols * wn + 32 * nt;  // uniform
      if (nbase >= N || rows <= 0) continue;
      int s = 0;
#pragma unroll
      for (int i = 1; i < kMaxLinearSegs; ++i)
        if (i < out.nseg && nbase >= out.col_begin[i]) s = i;
      const int ncol = N - nbase < 32 ? N - nbase : 32;
      if (ln >= ncol) continue;
      const int64_t stride = out.row_stride[s];
      const bool f32 = out.dtype[s] == kLinF32;
      const int esz = f32 ? 4 : 2;
      const __amdgpu_buffer_rsrc_t ro = rsrc(
          (char *)out.ptr[s] + (r0 * stride + (nbase - out.col_begin[s])) * esz,
          (uint32_t)(((rows - 1) * stride + ncol) * esz));
      const uint32_t vo = (uint32_t)((4 * lh * stride + ln) * esz);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t so = (uint32_t)((32 * mt + 8 * (r >> 2) + (r & 3)) * stride * esz);
          const float x = acc[mt][nt][r];
          if (f32)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), ro, vo, so, 0);
          else
            __builtin_amdgcn_raw_buffer_store_b16(f2bf(x), ro, vo, so, 0);
        }
    }
  } else {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int nbase = n0 + kWaveCols * wn + 32 * nt;
      if (nbase >= N) continue;
      const int col = nbase + (lane & 31);
      if (col >= N) continue;
      int s = 0;  // the lane's column's segment
#pragma unroll
      for (int i = 1; i < kMaxLinearSegs; ++i)
        if (i < out.nseg && col >= out.col_begin[i]) s = i;
      const int64_t cs = col - out.col_begin[s];
      const int64_t stride = out.row_stride[s];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = m0 + kWaveRows * wm + 32 * mt + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (row >= M) continue;
          const float x = acc[mt][nt][r];
          if (out.dtype[s] == kLinF32)
            reinterpret_cast<float *>(out.ptr[s])[row * stride + cs] = x;
          else
            reinterpret_cast<bf16_t *>(out.ptr[s])[row * stride + cs] = f2bf(x);
        }
      }
    }
  }
}

}  // namespace

size_t linear_lds_bytes() { return kLinLds; }

hipError_t launch_linear_bf16(const void *A, const void *W, int64_t M, int N, int K,
                              const LinearOut &out, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  bool tile_seg = true;
  for (int i = 0; i < out.nseg; ++i) {
    if (out.col_begin[i] % 32 != 0) tile_seg = false;
    // the buffer-store epilogue also needs the row strides to fit its 32-bit offsets
    if (out.row_stride[i] > (int64_t)1 << 22) tile_seg = false;
  }
  static std::atomic<uint64_t> lds_set[2];
  const void *fn = tile_seg ? (const void *)linear_bf16_kernel<true>
                            : (const void *)linear_bf16_kernel<false>;
  if (hipError_t e = ensure_lds_limit(fn, (int)kLinLds, lds_set[tile_seg]); e != hipSuccess)
    return e;
  const int64_t blocks = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  if (tile_seg)
    hipLaunchKernelGGL(linear_bf16_kernel<true>, dim3((unsigned)blocks), dim3(kLinThreads), kLinLds,
                       stream, (const bf16_t *)A, (const bf16_t *)W, M, N, K, out);
  else
    hipLaunchKernelGGL(linear_bf16_kernel<false>, dim3((unsigned)blocks), dim3(kLinThreads),
                       kLinLds, stream, (const bf16_t *)A, (const bf16_t *)W, M, N, K, out);
  return hipGetLastError();
}

}  // namespace gdn
