// kq_mfma.hip — matrix-core variant: each block's transform as a small matrix
// product on the matrix cores (KroQuant abstract: the per-block transforms map
// onto small matrix-unit products).
//
// For a 32-channel block b and 32 token rows, Y_b^T (32 channels x 32 tokens) =
// T_b (32x32) * X_b^T (32 x 32 tokens) on v_mfma_f32_32x32x16_bf16 with fp32
// accumulation.  T_b is given as three bf16 parts hi + mid + lo that sum exactly
// to its fp32 entries (kq_expand_factors, KQ_T_DENSE_BF16X3); bf16 x bf16 products
// are exact in fp32, so the three-pass product carries fp32 accuracy in T.  The
// input must be bf16 (its values are exact MFMA operands).
//
// Operand layout of the 32x32x16 bf16 MFMA (wave64): lane l supplies 8 consecutive
// K values k = 8*(l/32) .. +7 of row (A) / column (B) l%32; the 16 fp32 results of
// lane l are column l%32, rows 8*g + 4*(l/32) + r (g, r = 0..3).  With A = T_b rows
// and B = token columns, each lane therefore holds 16 channels of one token, the
// other 16 sit in lane l^32: the block amax and the packed code bytes are completed
// with one cross-half exchange each.
//
// Data flow.  A workgroup (4 waves) owns a group of 8 adjacent blocks and walks
// 32-row tiles of them (32 rows x 512 contiguous bytes).  Its 256 threads load a
// tile with fully coalesced 16-byte accesses into registers one tile ahead, park
// it in LDS (double-buffered, 528-byte row pitch so the 32 rows of a column fall
// on distinct banks) and each wave reads its two blocks' MFMA operands back with
// ds_read_b128.  The 12 A operands of a wave's two blocks stay in VGPRs for the
// whole walk.  The code bytes of a tile are staged in LDS and leave as whole
// 128-byte row segments (written straight from the lanes they would be 16-byte
// pieces of 32 rows per instruction, partial lines).  Rows past the end and blocks
// past nb are clamped to the last row / block: those lanes recompute and re-store
// exactly the bytes of the lane that owns them, so no memory operation is
// predicated.
#include "kq_device.hpp"
#include "kq_launch.hpp"

// Products and sums round separately unless written as an explicit fma.
#pragma clang fp contract(off)

namespace kq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTileRows = 32;
constexpr int kTileBlocks = 8;                    // 2 per wave
constexpr int kChunksPerRow = kTileBlocks * 4;    // 16-byte chunks per tile row
constexpr int kPitch = kTileBlocks * 64 + 16;     // LDS row pitch in bytes
constexpr int kTileBytes = kTileRows * kPitch;
constexpr int kChunksPerThread = kTileRows * kChunksPerRow / kThreads;  // 4
constexpr int kQPitch = kTileBlocks * 16 + 16;    // staged code row: 128 bytes + 16
static_assert(kTileRows * kTileBlocks * 16 == kThreads * 16, "one 16-byte code store per thread");

constexpr int kMfmaBlocksPerCU = 3;  // resident workgroups per CU (LDS: 38 KB each)

// Encodes one block of one token (this lane's half of it): the 16 code bytes go to
// the workgroup's staging row `qrow` in LDS, the scale byte straight to memory.
template <bool WRITE_Y>
__device__ __forceinline__ void encode_tile(floatx16 acc, int h, uint8_t* qrow, uint8_t* srow,
                                            float* yrow) {
  float m = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; r += 2) m = amax3(m, acc[r], acc[r + 1]);
  m = __builtin_elementwise_maximum(m, __shfl_xor(m, 32));
  if (WRITE_Y) {
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<float4*>(yrow + 8 * g + 4 * h) =
          make_float4(acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]);
  }
  const uint32_t S = e8m0_of_amax(m);
  uint32_t Sc = S;
  if (__builtin_expect(S < 25u, 0)) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] *= 0x1p64f;
    Sc = S + 64u;
  }
  const float sc = __uint_as_float(Sc << 23);
  // lane half h holds channels 8g + 4h + (0..3): code bytes 4g + 2h and 4g + 2h + 1
  uint32_t w0 = 0, w1 = 0;
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, acc[0], acc[1], sc, 0);
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, acc[2], acc[3], sc, 1);
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, acc[4], acc[5], sc, 2);
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, acc[6], acc[7], sc, 3);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, acc[8], acc[9], sc, 0);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, acc[10], acc[11], sc, 1);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, acc[12], acc[13], sc, 2);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, acc[14], acc[15], sc, 3);
  if (S == 255u) w0 = w1 = 0u;
  // h = 0 holds bytes {0,1,4,5 | 8,9,12,13}, h = 1 holds {2,3,6,7 | 10,11,14,15}:
  // lane h = 0 takes the other half's two words and stores the 16 bytes in one
  // piece (16-byte stores of 32 rows at the 144-byte pitch meet no LDS bank twice;
  // 8-byte stores from both halves put rows n and n + 8 on the same banks)
  const uint32_t r0 = (uint32_t)__shfl_xor((int)w0, 32), r1 = (uint32_t)__shfl_xor((int)w1, 32);
  if (h == 0) {
    const uint32_t b0 = (w0 & 0xFFFFu) | (r0 << 16), b1 = (w0 >> 16) | (r0 & 0xFFFF0000u);
    const uint32_t b2 = (w1 & 0xFFFFu) | (r1 << 16), b3 = (w1 >> 16) | (r1 & 0xFFFF0000u);
    *reinterpret_cast<u32x4*>(qrow) = u32x4{b0, b1, b2, b3};
    *srow = (uint8_t)S;
  }
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <bool WRITE_Y>
__global__ __launch_bounds__(kThreads) void mfma_kernel(
    const uint16_t* __restrict__ x, int64_t rows, uint32_t nb, int64_t ldx,
    const uint16_t* __restrict__ T3, uint8_t* __restrict__ q, int64_t ldq,
    uint8_t* __restrict__ s, int64_t lds, float* __restrict__ y, int64_t ldy, uint32_t tstep) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[2][kTileBytes];
  // the tile's code bytes, 32 rows of the group's 8 blocks (16 bytes each), padded
  __shared__ __attribute__((aligned(16))) uint8_t qstage[kTileRows][kQPitch];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h = lane >> 5;
  // the grid is a multiple of the block-group count (tstep tiles per pass)
  const uint32_t ngroups = (nb + kTileBlocks - 1) / kTileBlocks;
  const uint32_t bg = blockIdx.x % ngroups;
  uint32_t rt = blockIdx.x / ngroups;
  const uint32_t ntiles = (uint32_t)((rows + kTileRows - 1) / kTileRows);
  if (rt >= ntiles) return;
  const int64_t last = rows - 1;

  // this thread's 4 tile chunks: rows (tid/32) + 8 i, chunk column tid % 32
  const int ccol = tid & (kChunksPerRow - 1);
  uint32_t cblk = bg * kTileBlocks + (ccol >> 2);
  if (cblk > nb - 1) cblk = nb - 1;
  const int64_t ccol_elem = (int64_t)cblk * kBlk + (ccol & 3) * 8;
  const int crow0 = tid / kChunksPerRow;
  // (register-friendly vector type: an array of HIP's uint4 struct ends up in
  // scratch memory, each load waited for at once)
  u32x4 R[kChunksPerThread];
  auto load_tile = [&](uint32_t t_idx) {
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i) {
      int64_t row = (int64_t)t_idx * kTileRows + crow0 + 8 * i;
      row = row < last ? row : last;
      R[i] = *reinterpret_cast<const u32x4*>(x + row * ldx + ccol_elem);
    }
  };
  load_tile(rt);

  // A operands of this wave's two blocks: [block][split hi/mid/lo][K half]
  uint32_t blk[2];
  bf16x8 A[2][3][2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint32_t b = bg * kTileBlocks + 2 * wave + j;
    blk[j] = b < nb ? b : nb - 1;
#pragma unroll
    for (int sp = 0; sp < 3; ++sp)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
        A[j][sp][kh] = *reinterpret_cast<const bf16x8*>(
            T3 + ((size_t)sp * nb + blk[j]) * 1024 + n * 32 + 16 * kh + 8 * h);
  }

  int buf = 0;
  for (;;) {
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i)
      *reinterpret_cast<u32x4*>(&tile[buf][(crow0 + 8 * i) * kPitch + ccol * 16]) = R[i];
    __syncthreads();
    const uint32_t rn = rt + tstep;
    // next tile in flight during the math (clamped: the last pass re-reads a valid tile)
    load_tile(rn < ntiles ? rn : rt);

    int64_t t = (int64_t)rt * kTileRows + n;
    t = t < last ? t : last;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int jb = 2 * wave + j;
      const uint8_t* src = &tile[buf][n * kPitch + jb * 64 + 16 * h];
      const bf16x8 B0 = as_bf16x8(*reinterpret_cast<const u32x4*>(src));
      const bf16x8 B1 = as_bf16x8(*reinterpret_cast<const u32x4*>(src + 32));
      floatx16 acc = {};
      // smallest parts first
#pragma unroll
      for (int sp = 2; sp >= 0; --sp) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[j][sp][0], B0, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[j][sp][1], B1, acc, 0, 0, 0);
      }
      encode_tile<WRITE_Y>(acc, h, &qstage[n][16 * jb], s + t * lds + blk[j],
                           WRITE_Y ? y + t * ldy + 32 * blk[j] : nullptr);
    }
    __syncthreads();
    // the tile's codes leave as whole 128-byte row segments: 8 threads per row, each
    // 16 bytes (rows past the end and blocks past nb hold exactly the bytes of the
    // last row / block, and are written there again)
    {
      const int sr = tid >> 3, sc = tid & 7;
      int64_t row = (int64_t)rt * kTileRows + sr;
      row = row < last ? row : last;
      uint32_t b = bg * kTileBlocks + sc;
      b = b < nb ? b : nb - 1;
      const u32x4 v = *reinterpret_cast<const u32x4*>(&qstage[sr][16 * sc]);
      *reinterpret_cast<u32x4*>(q + row * ldq + 16 * b) = v;
    }
    if (rn >= ntiles) return;
    rt = rn;
    buf ^= 1;
  }
}

template <bool WRITE_Y>
hipError_t launch_t(const LaunchArgs& a) {
  const int64_t ngroups = (a.nb + kTileBlocks - 1) / kTileBlocks;
  const int64_t ntiles = (a.rows + kTileRows - 1) / kTileRows;
  int64_t target = (int64_t)a.cus * kMfmaBlocksPerCU;
  if (target > ngroups * ntiles) target = ngroups * ntiles;
  int64_t k = (target + ngroups - 1) / ngroups;
  if (k < 1) k = 1;
  hipLaunchKernelGGL((mfma_kernel<WRITE_Y>), dim3((unsigned)(k * ngroups)), dim3(kThreads), 0,
                     (hipStream_t)a.stream, (const uint16_t*)a.x, a.rows, (uint32_t)a.nb, a.ldx,
                     (const uint16_t*)a.t, a.q, a.ldq, a.s, a.lds, a.y, a.ldy, (uint32_t)k);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma(const LaunchArgs& a) {
  return a.y ? launch_t<true>(a) : launch_t<false>(a);
}

}  // namespace kq
