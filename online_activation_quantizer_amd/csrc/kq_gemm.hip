// kq_gemm.hip — the W4A4 product that consumes the quantizer's output (gfx950).
//
//   Y[m][n] = sum_k deq(A)[m][k] * deq(B)[n][k]
//
// A = the activations' MXFP4 codes and E8M0 scales exactly as kq_quantize writes
// them ([M][K/2] code bytes, [M][K/32] scale bytes), B = the weights' (as
// kq_quantize_weights writes them, [N][K/2] and [N][K/32]).  KroQuant abstract:
// W4A4 with MXFP4 activations and weights; the transform's inverse folded into the
// weights makes this product equal W x up to the two quantizations.
//
// Matrix cores.  v_mfma_scale_f32_32x32x64_f8f6f4 with both operands in fp4
// (E2M1) multiplies a 32x64 by a 64x32 tile and applies one E8M0 scale per 32
// K-values of each row (OCP MX block size) in hardware, accumulating in fp32.  Lane
// l supplies row l % 32 and the 32 K-values 32 (l / 32) .. + 31 as 16 bytes, low
// nibble first, which is exactly one 32-element block of the quantizer's layout,
// plus that block's scale byte (chosen from a 32-bit register by op_sel).
//
// Tiling.  A workgroup (4 waves, 2 x 2) computes a 128 x 128 tile of Y; each wave a
// 64 x 64 quarter as 2 x 2 MFMA tiles.  K advances 64 KSUB values at a time (256 by
// default: 128 code bytes per row, whole cache lines): the code tiles of A and B
// and their scale bytes are staged through LDS (double-buffered, code rows padded
// by 16 bytes against bank conflicts), with the global loads of the step after
// next in flight during this step's MFMAs.  Rows past M or N are clamped on load
// and not stored; K-blocks past K get scale 2^-127 on both operands (their
// products vanish).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kq_launch.hpp"

namespace kq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));  // register-friendly 16 bytes
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kBM = 128, kBN = 128;

#ifndef KQ_GEMM_KSUB
#define KQ_GEMM_KSUB 4
#endif
// 64-element K substeps (one MFMA each) per staged K step: K step = 64 KSUB values,
// 32 KSUB code bytes per row
constexpr int kKSub = KQ_GEMM_KSUB;
constexpr int kBKBytes = 32 * kKSub;
constexpr int kPitch = kBKBytes + 16;      // LDS code-row pitch (bank spread)
constexpr int kTileCodes = 128 * kPitch;   // bytes per operand per stage
constexpr int kChunks = kKSub;             // 16-byte code chunks per thread per operand
constexpr int kScaleWords = kKSub / 2;     // 32-bit scale words per row per step

struct Stage {
  u32x4 a[kChunks], b[kChunks];  // this thread's code chunks of A and of B
  uint32_t sc[kScaleWords];      // one row's scale bytes (threads 0-127: A, 128-255: B)
};

template <bool OUT_BF16, bool SCALE_WORDS>
__global__ __launch_bounds__(256) void mx_gemm_kernel(
    const uint8_t* __restrict__ qa, uint32_t lda, const uint8_t* __restrict__ sa, uint32_t ldsa,
    const uint8_t* __restrict__ qb, uint32_t ldb, const uint8_t* __restrict__ sb, uint32_t ldsb,
    uint32_t M, uint32_t N, uint32_t K, void* __restrict__ out, uint32_t ldo, uint32_t tiles_n,
    uint32_t xcd_cols) {
  __shared__ __attribute__((aligned(16))) uint8_t codes[2][2][kTileCodes];  // [stage][A/B]
  __shared__ uint32_t scales[2][2][128][kScaleWords];
  const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
  const uint32_t wm = wave >> 1, wn = wave & 1u;
  // Tile order.  Workgroups go to the 8 XCDs round-robin by index; when xcd_cols > 0
  // (tiles_n = 8 xcd_cols) XCD x gets the tile columns [x xcd_cols, (x+1) xcd_cols)
  // for every tile row, so the B tiles it reads stay in its own L2 while the tile
  // rows advance, and consecutive workgroups on an XCD share their A tile.
  uint32_t tm, tn;
  if (xcd_cols) {
    const uint32_t x = blockIdx.x & 7u, local = blockIdx.x >> 3;
    tm = local / xcd_cols;
    tn = x * xcd_cols + (local - tm * xcd_cols);
  } else {
    tm = blockIdx.x / tiles_n;
    tn = blockIdx.x - tm * tiles_n;
  }
  const uint32_t m0 = tm * kBM, n0 = tn * kBN;
  const uint32_t kbytes = K / 2, kblocks = K / 32;
  const uint32_t nsteps = (K + 64 * kKSub - 1) / (64 * kKSub);

  // global -> register loads of one K step.  No load sits under a branch (the
  // compiler would then wait for every load in flight): code chunks past K re-read
  // the row's last chunk, and their scale bytes on both operands are 0x00 (2^-127),
  // so each of their products is below 36 * 2^-254 and vanishes in the fp32
  // accumulation whatever the codes (E2M1 codes are all finite).
  auto load_stage = [&](uint32_t step, Stage& st) {
    const uint32_t kb0 = step * kBKBytes;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      // chunk c: row c / (2 KSUB), 16-byte column c % (2 KSUB)
      const uint32_t c = tid + 256u * i;
      const uint32_t row = c / (2 * kKSub), col = (c % (2 * kKSub)) * 16u;
      const uint32_t off = kb0 + col < kbytes ? kb0 + col : kbytes - 16u;
      const uint32_t ra = m0 + row < M ? m0 + row : M - 1;
      const uint32_t rb = n0 + row < N ? n0 + row : N - 1;
      st.a[i] = *reinterpret_cast<const u32x4*>(qa + (uint64_t)ra * lda + off);
      st.b[i] = *reinterpret_cast<const u32x4*>(qb + (uint64_t)rb * ldb + off);
    }
    // scales: thread t < 128 takes A row t, t >= 128 takes B row t - 128
    const bool isb = tid >= 128u;
    const uint32_t row = tid & 127u;
    const uint32_t r = isb ? (n0 + row < N ? n0 + row : N - 1) : (m0 + row < M ? m0 + row : M - 1);
    const uint32_t blk0 = step * 2u * kKSub;  // first scale byte of this step
    const uint8_t* srow = isb ? sb + (uint64_t)r * ldsb : sa + (uint64_t)r * ldsa;
#pragma unroll
    for (int wdx = 0; wdx < kScaleWords; ++wdx) {
      const uint32_t b0 = blk0 + 4u * wdx;
      const uint32_t valid = b0 < kblocks ? kblocks - b0 : 0u;  // bytes of this word inside K
      const uint32_t keep = valid >= 4u ? 0xFFFFFFFFu : (1u << (8u * valid)) - 1u;
      uint32_t w;
      if (SCALE_WORDS) {
        // kblocks >= 4 here: read the last whole word when this one runs past the end
        const uint32_t at = b0 + 4u <= kblocks ? b0 : kblocks - 4u;
        const uint32_t raw = *reinterpret_cast<const uint32_t*>(srow + at);
        const uint32_t sh = 8u * (b0 - at);  // 0 .. 24, or >= 32 wholly past the end
        w = sh < 32u ? raw >> sh : 0u;
      } else {
        // byte by byte from clamped addresses (no load under a branch)
        w = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t at = b0 + j < kblocks ? b0 + j : kblocks - 1u;
          w |= (uint32_t)srow[at] << (8 * j);
        }
      }
      st.sc[wdx] = w & keep;  // bytes past K: 0x00
    }
  };
  auto store_stage = [&](int buf, const Stage& st) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const uint32_t c = tid + 256u * i;
      const uint32_t off = (c / (2 * kKSub)) * kPitch + (c % (2 * kKSub)) * 16u;
      *reinterpret_cast<u32x4*>(&codes[buf][0][off]) = st.a[i];
      *reinterpret_cast<u32x4*>(&codes[buf][1][off]) = st.b[i];
    }
#pragma unroll
    for (int wdx = 0; wdx < kScaleWords; ++wdx) scales[buf][tid >> 7][tid & 127u][wdx] = st.sc[wdx];
  };

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};

  const uint32_t lr = lane & 31u, h = lane >> 5;
  // step s is computed from LDS while step s + 1 waits in registers for its LDS
  // slot and step s + 2 is in flight from memory
  Stage nxt, far;
  load_stage(0, nxt);
  store_stage(0, nxt);
  if (nsteps > 1) load_stage(1, nxt);
  __syncthreads();
  int buf = 0;
  for (uint32_t step = 0; step < nsteps; ++step) {
    if (step + 2 < nsteps) load_stage(step + 2, far);
#pragma unroll
    for (int ks = 0; ks < kKSub; ++ks) {
      v8i A[2], B[2];
      uint32_t sA[2], sB[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t ra = wm * 64u + 32u * i + lr, rb = wn * 64u + 32u * i + lr;
        const u32x4 va = *reinterpret_cast<const u32x4*>(&codes[buf][0][ra * kPitch + 32u * ks + 16u * h]);
        const u32x4 vb = *reinterpret_cast<const u32x4*>(&codes[buf][1][rb * kPitch + 32u * ks + 16u * h]);
        A[i] = v8i{(int)va.x, (int)va.y, (int)va.z, (int)va.w, 0, 0, 0, 0};
        B[i] = v8i{(int)vb.x, (int)vb.y, (int)vb.z, (int)vb.w, 0, 0, 0, 0};
        // the lane's block scale (byte 2 ks + h of the row's step) moved to byte
        // 2 (ks % 2) of its word, which op_sel picks
        sA[i] = scales[buf][0][ra][ks / 2] >> (8u * h);
        sB[i] = scales[buf][1][rb][ks / 2] >> (8u * h);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if (ks % 2 == 0)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                A[i], B[j], acc[i][j], 4, 4, 0, (int)sA[i], 0, (int)sB[j]);
          else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                A[i], B[j], acc[i][j], 4, 4, 2, (int)sA[i], 2, (int)sB[j]);
        }
    }
    // keep the next step's LDS stores (and their wait for its loads) after this
    // step's products
    __builtin_amdgcn_sched_barrier(0);
    if (step + 1 < nsteps) {
      // the other slot was last read before the previous barrier
      store_stage(buf ^ 1, nxt);
      // field by field (a struct copy here ends up in scratch memory)
#pragma unroll
      for (int i = 0; i < kChunks; ++i) {
        nxt.a[i] = far.a[i];
        nxt.b[i] = far.b[i];
      }
#pragma unroll
      for (int wdx = 0; wdx < kScaleWords; ++wdx) nxt.sc[wdx] = far.sc[wdx];
      __syncthreads();
      buf ^= 1;
    }
  }

  // acc[i][j][r]: row 8 (r / 4) + 4 h + r % 4 of MFMA tile (i, j), column lr
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t col = n0 + wn * 64u + 32u * j + lr;
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t row = m0 + wm * 64u + 32u * i + 8u * (r >> 2) + 4u * h + (r & 3);
        if (row >= M) continue;
        if (OUT_BF16) {
          const float v = acc[i][j][r];
          // round to nearest even (finite values)
          const uint32_t u = __float_as_uint(v);
          const uint16_t hb = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
          // streaming stores: Y is not re-read here and must not evict the operand tiles
          __builtin_nontemporal_store(hb, reinterpret_cast<uint16_t*>(out) + (uint64_t)row * ldo + col);
        } else {
          __builtin_nontemporal_store(acc[i][j][r], reinterpret_cast<float*>(out) + (uint64_t)row * ldo + col);
        }
      }
    }
}

}  // namespace

template <bool OUT_BF16, bool SCALE_WORDS>
void launch_t(const GemmArgs& g, int64_t grid, int64_t tiles_n, int64_t xcd_cols) {
  hipLaunchKernelGGL((mx_gemm_kernel<OUT_BF16, SCALE_WORDS>), dim3((unsigned)grid), dim3(256), 0,
                     (hipStream_t)g.stream, g.qa, (uint32_t)g.lda, g.sa, (uint32_t)g.ldsa, g.qb,
                     (uint32_t)g.ldb, g.sb, (uint32_t)g.ldsb, (uint32_t)g.M, (uint32_t)g.N,
                     (uint32_t)g.K, g.out, (uint32_t)g.ldo, (uint32_t)tiles_n, (uint32_t)xcd_cols);
}

hipError_t launch_mx_gemm(const GemmArgs& g) {
  const int64_t tiles_m = (g.M + kBM - 1) / kBM, tiles_n = (g.N + kBN - 1) / kBN;
  const int64_t grid = tiles_m * tiles_n;
  const int64_t xcd_cols = tiles_n % 8 == 0 ? tiles_n / 8 : 0;
  // whole 32-bit scale words when every scale row starts 4-byte aligned and holds one
  const bool words = ((uintptr_t)g.sa % 4 == 0) && ((uintptr_t)g.sb % 4 == 0) && g.ldsa % 4 == 0 &&
                     g.ldsb % 4 == 0 && g.K >= 128;
  if (g.out_bf16) {
    if (words) launch_t<true, true>(g, grid, tiles_n, xcd_cols);
    else launch_t<true, false>(g, grid, tiles_n, xcd_cols);
  } else {
    if (words) launch_t<false, true>(g, grid, tiles_n, xcd_cols);
    else launch_t<false, false>(g, grid, tiles_n, xcd_cols);
  }
  return hipGetLastError();
}

}  // namespace kq
