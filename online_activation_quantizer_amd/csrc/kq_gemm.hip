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
// plus that block's scale byte (chosen from a 32-bit register by op_sel).  The
// weight tile goes in as the instruction's first operand and the activation tile as
// its second, so the product comes out transposed: lane l holds row l % 32 of Y and
// four consecutive columns per register quad, stored as one 8-byte (bf16) or
// 16-byte (fp32) write.
//
// Tiling.  A workgroup of 8 waves (2 x 4) computes 256 x 256 tiles of Y, each wave
// a 128 x 64 part as 4 x 2 MFMA tiles (reading 0.75 KB of LDS per MFMA).  K
// advances 256 values per step (128 code bytes per row, whole cache lines): the code
// tiles of A and B and their scale bytes are staged through LDS (two slots, code rows
// padded by 16 bytes against bank conflicts; 152 KB), from one register stage whose
// global loads run a step ahead; its LDS stores go out one by one between the first
// substep's products.  The grid is persistent (one workgroup per compute unit,
// tiles strided by the grid), and the step sequence runs across tile boundaries:
// the next tile's first steps load while a tile's last step multiplies and its
// outputs are written.  Code rows past M or N read zeros (buffer loads through a
// per-tile range) and are not stored; K-blocks past K get scale 2^-127 on both
// operands (their products vanish).
//
// Split tiles.  With a workspace and few tiles (at most half the compute units
// busy) and a long K, each tile is computed as S parts of K on S workgroups of its
// XCD; every part but the last to finish stores its fp32 sums, and the last adds
// all parts in part order and writes the tile (kernel variant SPLIT).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "kq_launch.hpp"
#include "kq_split.hpp"

namespace kq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));  // register-friendly 16 bytes
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

// 64-element K substeps (one MFMA each) per staged K step: K step = 256 values, 128
// code bytes per row
constexpr int kKSub = 4;
constexpr int kBKBytes = 32 * kKSub;
constexpr int kRowChunks = kBKBytes / 16;  // 16-byte code chunks per row per step
constexpr int kPitch = kBKBytes + 16;      // LDS code-row pitch (bank spread)
constexpr int kScaleWords = kKSub / 2;     // 32-bit scale words per row per step

// Workgroup tiling: WAVES_M x WAVES_N waves, each computing TM x TN tiles of 32 x 32.
template <int WAVES_M, int WAVES_N, int TM, int TN>
struct Tiling {
  static constexpr int kWavesN = WAVES_N, kTM = TM, kTN = TN;
  static constexpr int kThreads = 64 * WAVES_M * WAVES_N;
  static constexpr int kBM = 32 * TM * WAVES_M, kBN = 32 * TN * WAVES_N;
  static constexpr int kRows = kBM + kBN;  // LDS rows per slot: A's, then B's
  static constexpr int kChunks = kRows * kRowChunks / kThreads;  // code chunks per thread
  static constexpr int kChunksA = kBM * kRowChunks / kThreads;   // of which from A
  static constexpr int kScaleRows = (kRows + kThreads - 1) / kThreads;
  static_assert(kBM * kRowChunks % kThreads == 0 && kBN * kRowChunks % kThreads == 0,
                "each thread's code chunks must split evenly between the operands");
  static_assert(kThreads % kRowChunks == 0, "a thread keeps its chunk column across rows");
  // staged output: each wave's 32 TM x 64 part goes through a 64-row region of one
  // LDS slot (64 code-row pitches per wave)
  static constexpr bool kCanStage = TN == 2 && TM % 2 == 0 && WAVES_M * WAVES_N * 64 * kPitch <= kRows * kPitch;
};

// 256 x 256 tiles, 8 waves of 128 x 64
using ProductTiling = Tiling<2, 4, 4, 2>;

// One K step of this thread's share of both operands, as loaded (scale words are
// shifted and masked when stored to LDS, so no arithmetic waits on a load early).
template <class T, bool SCALE_WORDS>
struct Stage {
  u32x4 c[T::kChunks];                                          // code chunks
  uint32_t sc[T::kScaleRows][kScaleWords * (SCALE_WORDS ? 1 : 4)];  // scale words (or bytes)
};

// Output paths (EPI): kEpiScalar one output per store; kEpiVec4 four consecutive
// outputs per store straight from the accumulators (N and ldo multiples of 4, output
// 8- or 16-byte aligned); kEpiStaged (bf16 only; N and ldo multiples of 8, output
// 16-byte aligned) the tile goes through LDS so that each store instruction writes
// whole 128-byte row segments.
constexpr int kEpiScalar = 0, kEpiVec4 = 1, kEpiStaged = 2;

// marks a tile written from its accumulators alone
struct NoPartial {};

// the most K parts a split tile runs in (the exchange loads one slot per part)
constexpr int kSplitMaxPartsDev = 8;


template <class T, bool OUT_BF16, int EPI, bool SCALE_WORDS, bool SPLIT>
__global__ __launch_bounds__(T::kThreads) __attribute__((amdgpu_waves_per_eu(2))) void mx_gemm_kernel(
    const uint8_t* __restrict__ qa, uint32_t lda, const uint8_t* __restrict__ sa, uint32_t ldsa,
    const uint8_t* __restrict__ qb, uint32_t ldb, const uint8_t* __restrict__ sb, uint32_t ldsb,
    uint32_t M, uint32_t N, uint32_t K, void* __restrict__ out, uint32_t ldo, uint32_t tiles_n,
    uint32_t ntiles, uint32_t xcd_cols, uint32_t band_rows, uint32_t parts, uint32_t* __restrict__ flags,
    float* __restrict__ partials) {
  constexpr int kRows = T::kRows, kBM = T::kBM, kThreads = T::kThreads;
  static_assert(EPI != kEpiStaged || (OUT_BF16 && T::kCanStage), "staged output: bf16, tiles that fit");
  __shared__ __attribute__((aligned(16))) uint8_t codes[2][kRows * kPitch];  // [slot], A rows then B rows
  __shared__ __attribute__((aligned(8))) uint32_t scales[2][kRows][kScaleWords];
  const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
  const uint32_t wm = wave / T::kWavesN, wn = wave % T::kWavesN;
  const uint32_t grid = gridDim.x;
  const uint32_t kbytes = K / 2, kblocks = K / 32;
  const uint32_t nsteps = (K + 64 * kKSub - 1) / (64 * kKSub);

  // Tile t -> first row and column.  Workgroups go to the 8 XCDs round-robin by
  // index and the grid is a multiple of 8, so all tiles of a workgroup share
  // t % 8; when xcd_cols > 0 (tiles_n = 8 xcd_cols) XCD x gets the tile columns
  // [x xcd_cols, (x+1) xcd_cols) for every tile row, so the B tiles it reads stay in
  // its own L2 while the tile rows advance, and workgroups running together on an
  // XCD share their A tiles.  SPLIT: each XCD's tiles form one compact block of the
  // tile grid (split_tile).
  auto tile_origin = [&](uint32_t t, uint32_t& m0, uint32_t& n0) {
    if constexpr (SPLIT) {
      uint32_t tm, tn;
      split_tile(t, ntiles, tiles_n, band_rows, tm, tn);
      m0 = tm * kBM;
      n0 = tn * T::kBN;
      return;
    }
    // (selects, no branch: with xcd_cols = 0 this is tm = t / tiles_n, tn = t % tiles_n)
    const uint32_t per = xcd_cols ? xcd_cols : tiles_n;
    const uint32_t x = xcd_cols ? t & 7u : 0u, local = xcd_cols ? t >> 3 : t;
    const uint32_t tm = local / per;
    const uint32_t tn = x * per + (local - tm * per);
    m0 = tm * kBM;
    n0 = tn * T::kBN;
  };

  // The rows this thread loads for the tile being fetched (origin lm0, ln0): code
  // chunk i is LDS row (tid + kThreads i) / kRowChunks (the first kChunksA of them A
  // rows), scale row j is LDS row tid + kThreads j (past the last row a duplicate
  // whose value is not stored).  Code chunks are buffer loads through one descriptor
  // per operand whose range ends with the tile's last row inside the matrix (K
  // codes in): chunks of rows past M or N read zeros, and their products are not
  // stored.  Scale rows past M or N re-read the matrix's last row.
  uint32_t lm0 = 0, ln0 = 0;
  __amdgpu_buffer_rsrc_t rsrc_a, rsrc_b;
  auto set_rows = [&](uint32_t t) {
    tile_origin(t, lm0, ln0);
    const uint32_t rows_a = M - lm0 < (uint32_t)kBM ? M - lm0 : (uint32_t)kBM;
    const uint32_t rows_b = N - ln0 < (uint32_t)T::kBN ? N - ln0 : (uint32_t)T::kBN;
    rsrc_a = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(qa) + (uint64_t)lm0 * lda, 0,
                                               (int)((rows_a - 1u) * lda + kbytes), 0x00020000);
    rsrc_b = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(qb) + (uint64_t)ln0 * ldb, 0,
                                               (int)((rows_b - 1u) * ldb + kbytes), 0x00020000);
  };
  // byte offset of this thread's first code chunk in its A and B rows of a tile
  const uint32_t chunk_a = (tid / kRowChunks) * lda + 16u * (tid % kRowChunks);
  const uint32_t chunk_b = (tid / kRowChunks) * ldb + 16u * (tid % kRowChunks);
  auto scale_row = [&](int j) -> const uint8_t* {
    const uint32_t r0 = tid + kThreads * j, r = r0 < (uint32_t)kRows ? r0 : kRows - 1;
    if (r < (uint32_t)kBM) {
      const uint32_t g = lm0 + r < M ? lm0 + r : M - 1;
      return sa + (uint64_t)g * ldsa;
    }
    const uint32_t g = ln0 + (r - kBM) < N ? ln0 + (r - kBM) : N - 1;
    return sb + (uint64_t)g * ldsb;
  };

  // global -> register loads of K step `step` of the current rows.  No load sits
  // under a branch (the compiler would then wait for every load in flight): code
  // chunks past K read the bytes after the row (the next row's, or zeros past the
  // descriptor's range), and their scale bytes on both operands become 0x00
  // (2^-127) when stored, so each of their products is below 36 * 2^-254 and
  // vanishes in the fp32 accumulation whatever the codes (E2M1 codes are finite).
  constexpr uint32_t kRowsPerChunk = kThreads / kRowChunks;  // LDS rows between chunks i and i + 1
  auto load_chunk = [&](uint32_t kb0, int i, Stage<T, SCALE_WORDS>& st) {
    if (i < T::kChunksA)
      st.c[i] = __builtin_amdgcn_raw_buffer_load_b128(rsrc_a, chunk_a + kRowsPerChunk * i * lda + kb0, 0, 0);
    else
      st.c[i] = __builtin_amdgcn_raw_buffer_load_b128(
          rsrc_b, chunk_b + kRowsPerChunk * (i - T::kChunksA) * ldb + kb0, 0, 0);
  };
  auto load_scales = [&](uint32_t step, Stage<T, SCALE_WORDS>& st) {
    const uint32_t blk0 = step * 2u * kKSub;  // first scale byte of this step
#pragma unroll
    for (int j = 0; j < T::kScaleRows; ++j) {
      const uint8_t* srow = scale_row(j);
#pragma unroll
      for (int wdx = 0; wdx < kScaleWords; ++wdx) {
        const uint32_t b0 = blk0 + 4u * wdx;
        if (SCALE_WORDS) {
          // kblocks >= 4 here: read the last whole word when this one runs past the end
          const uint32_t w_at = b0 + 4u <= kblocks ? b0 : kblocks - 4u;
          st.sc[j][wdx] = *reinterpret_cast<const uint32_t*>(srow + w_at);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t b_at = b0 + q < kblocks ? b0 + q : kblocks - 1u;
            st.sc[j][4 * wdx + q] = srow[b_at];
          }
        }
      }
    }
  };
  auto load_stage = [&](uint32_t step, Stage<T, SCALE_WORDS>& st) {
#pragma unroll
    for (int i = 0; i < T::kChunks; ++i) load_chunk(step * kBKBytes, i, st);
    load_scales(step, st);
  };
  auto store_chunk = [&](int slot, int i, const Stage<T, SCALE_WORDS>& st) {
    const uint32_t c = tid + kThreads * i;
    *reinterpret_cast<u32x4*>(&codes[slot][(c / kRowChunks) * kPitch + (c % kRowChunks) * 16u]) = st.c[i];
  };
  auto store_scales = [&](int slot, uint32_t step, const Stage<T, SCALE_WORDS>& st) {
    const uint32_t blk0 = step * 2u * kKSub;
#pragma unroll
    for (int j = 0; j < T::kScaleRows; ++j) {
      const uint32_t r = tid + kThreads * j;
#pragma unroll
      for (int wdx = 0; wdx < kScaleWords; ++wdx) {
        const uint32_t b0 = blk0 + 4u * wdx;
        const uint32_t valid = b0 < kblocks ? kblocks - b0 : 0u;  // bytes of this word inside K
        const uint32_t keep = valid >= 4u ? 0xFFFFFFFFu : (1u << (8u * valid)) - 1u;
        uint32_t w;
        if (SCALE_WORDS) {
          const uint32_t at = b0 + 4u <= kblocks ? b0 : kblocks - 4u;
          const uint32_t sh = 8u * (b0 - at);  // 0 .. 24, or >= 32 wholly past the end
          w = sh < 32u ? st.sc[j][wdx] >> sh : 0u;
        } else {
          w = st.sc[j][4 * wdx] | (st.sc[j][4 * wdx + 1] << 8) | (st.sc[j][4 * wdx + 2] << 16) |
              (st.sc[j][4 * wdx + 3] << 24);
        }
        if (kRows % kThreads == 0 || r < (uint32_t)kRows) scales[slot][r][wdx] = w & keep;  // past K: 0x00
      }
    }
  };
  auto store_stage = [&](int slot, uint32_t step, const Stage<T, SCALE_WORDS>& st) {
#pragma unroll
    for (int i = 0; i < T::kChunks; ++i) store_chunk(slot, i, st);
    store_scales(slot, step, st);
  };

  // acc[i][j]: the wave's A row tile i (32 rows of Y) times its B row tile j (32
  // columns of Y)
  v16f acc[T::kTM][T::kTN];
#pragma unroll
  for (int i = 0; i < T::kTM; ++i)
#pragma unroll
    for (int j = 0; j < T::kTN; ++j) acc[i][j] = v16f{};

  const uint32_t lr = lane & 31u, h = lane >> 5;
  // this step's 8 scale bytes of each of the wave's A and B row tiles (lane row lr)
  struct Scales {
    uint32_t a[T::kTM][kScaleWords], b[T::kTN][kScaleWords];
  };
  auto read_scales = [&](int slot, Scales& sc) {
#pragma unroll
    for (int i = 0; i < T::kTM; ++i) {
      const uint32_t r = wm * (32u * T::kTM) + 32u * i + lr;
#pragma unroll
      for (int w = 0; w < kScaleWords; ++w) sc.a[i][w] = scales[slot][r][w];
    }
#pragma unroll
    for (int j = 0; j < T::kTN; ++j) {
      const uint32_t r = kBM + wn * (32u * T::kTN) + 32u * j + lr;
#pragma unroll
      for (int w = 0; w < kScaleWords; ++w) sc.b[j][w] = scales[slot][r][w];
    }
  };
  // the products of one 64-wide K substep; after_mfma(u, acc) runs after the u-th
  auto compute_ks = [&](int slot, int ks, const Scales& sc, auto&& after_mfma) {
    v8i A[T::kTM], B[T::kTN];
#pragma unroll
    for (int i = 0; i < T::kTM; ++i) {
      const uint32_t r = wm * (32u * T::kTM) + 32u * i + lr;
      const u32x4 v = *reinterpret_cast<const u32x4*>(&codes[slot][r * kPitch + 32u * ks + 16u * h]);
      A[i] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < T::kTN; ++j) {
      const uint32_t r = kBM + wn * (32u * T::kTN) + 32u * j + lr;
      const u32x4 v = *reinterpret_cast<const u32x4*>(&codes[slot][r * kPitch + 32u * ks + 16u * h]);
      B[j] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < T::kTM; ++i)
#pragma unroll
      for (int j = 0; j < T::kTN; ++j) {
        // the lane's block scale (byte 2 ks + h of the row's step) moved to byte
        // 2 (ks % 2) of its word, which op_sel picks; B is the first operand
        const int sA = (int)(sc.a[i][ks / 2] >> (8u * h)), sB = (int)(sc.b[j][ks / 2] >> (8u * h));
        if (ks % 2 == 0)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(B[j], A[i], acc[i][j], 4, 4, 0, sB, 0, sA);
        else
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(B[j], A[i], acc[i][j], 4, 4, 2, sB, 2, sA);
        after_mfma(i * T::kTN + j, acc[i][j]);
      }
  };
  auto no_hook = [](int, const v16f&) {};

  // acc[i][j][4 q + e]: Y row lr of the wave's A tile i, column 8 q + 4 h + e of its
  // B tile j
  // `add` is NoPartial, or turns this workgroup's sums acc[i][j][4 q .. 4 q + 3]
  // into the whole split tile's (all K parts) as they are written
  auto outputs = [&](auto add, int i, int j, int q) -> f32x4 {
    const f32x4 v{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
    if constexpr (std::is_same_v<decltype(add), NoPartial>) return v;
    else return add(i, j, q, v);
  };
  auto write_tile = [&](uint32_t t, auto add) {
    uint32_t m0, n0;
    tile_origin(t, m0, n0);
#pragma unroll
    for (int i = 0; i < T::kTM; ++i) {
      const uint32_t row = m0 + wm * (32u * T::kTM) + 32u * i + lr;
      if (row >= M) continue;
#pragma unroll
      for (int j = 0; j < T::kTN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t col = n0 + wn * (32u * T::kTN) + 32u * j + 8u * q + 4u * h;
          const f32x4 v = outputs(add, i, j, q);
          if (OUT_BF16) {
            uint32_t b[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              // round to nearest even (finite values)
              const uint32_t u = __float_as_uint(v[e]);
              b[e] = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
            }
            uint16_t* p = reinterpret_cast<uint16_t*>(out) + (uint64_t)row * ldo + col;
            if (EPI == kEpiVec4) {
              if (col < N) *reinterpret_cast<u32x2*>(p) = u32x2{b[0] | (b[1] << 16), b[2] | (b[3] << 16)};
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (col + e < N) p[e] = (uint16_t)b[e];
            }
          } else {
            float* p = reinterpret_cast<float*>(out) + (uint64_t)row * ldo + col;
            if (EPI == kEpiVec4) {
              if (col < N) *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (col + e < N) p[e] = v[e];
            }
          }
        }
    }
  };

  // The tile through LDS slot `slot` (free at this point): each wave turns its 128 x
  // 64 part into bf16 rows in its own 64-row region of the slot (two halves), reads
  // them back as 16-byte pieces and stores them, 8 lanes per 128-byte row segment, so
  // every store instruction writes whole cache lines.  Only the wave's own lanes
  // share its region; one workgroup barrier at the end frees the slot for the next
  // step's operands.  The stores are buffer
  // stores whose descriptor spans the tile's rows of Y; pieces past N get an offset
  // outside it, so the hardware drops them with no branch.
  auto write_tile_staged = [&](uint32_t t, int slot, auto add) {
    uint32_t m0, n0;
    tile_origin(t, m0, n0);
    uint8_t* st = codes[slot] + wave * (64u * kPitch);
    const uint32_t rows = M - m0 < (uint32_t)kBM ? M - m0 : (uint32_t)kBM;  // rows of Y in this tile
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<uint16_t*>(out) + (uint64_t)m0 * ldo, 0, (int)(rows * ldo * 2u), 0x00020000);
#pragma unroll
    for (int half = 0; half < T::kTM / 2; ++half) {
#pragma unroll
      for (int ii = 0; ii < 2; ++ii)
#pragma unroll
        for (int j = 0; j < T::kTN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4 v = outputs(add, 2 * half + ii, j, q);
            uint32_t b[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              // round to nearest even (finite values)
              const uint32_t u = __float_as_uint(v[e]);
              b[e] = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
            }
            *reinterpret_cast<u32x2*>(st + (32u * ii + lr) * kPitch + (32u * j + 8u * q + 4u * h) * 2u) =
                u32x2{b[0] | (b[1] << 16), b[2] | (b[3] << 16)};
          }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t r = lane / 8u + 8u * k, c = lane % 8u;
        const u32x4 v = *reinterpret_cast<const u32x4*>(st + r * kPitch + c * 16u);
        const uint32_t row = wm * (32u * T::kTM) + 64u * half + r;  // in the tile
        const uint32_t col = n0 + wn * 64u + 8u * c;
        const uint32_t off = col < N ? (row * ldo + col) * 2u : 0x80000000u;
        __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, (int)off, 0, 0);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    // the next step stores its operands into this slot
    __syncthreads();
  };

  // The work of this workgroup.  Whole tiles: tiles blockIdx.x, + grid, ...
  // (my_tiles of them), nsteps K steps each.  SPLIT (fewer tiles than half the
  // grid): one K part of one tile, workgroup p n8 + t (n8 = ntiles rounded up to
  // 8, so all parts of a tile run on its XCD) taking steps
  // [p nsteps / parts, (p + 1) nsteps / parts) of tile t; workgroups past the
  // tiles have nothing to do.
  const uint32_t wg = blockIdx.x;
  uint32_t l_tile = wg, l_step = 0, l_end = nsteps;  // the step the next load fetches (split: [l_step, l_end))
  [[maybe_unused]] uint32_t part = 0;
  uint64_t total;
  if constexpr (SPLIT) {
    const uint32_t n8 = (ntiles + 7u) & ~7u;
    part = wg / n8;
    l_tile = wg - part * n8;
    if (l_tile >= ntiles || part >= parts) return;
    l_step = (uint32_t)((uint64_t)part * nsteps / parts);
    l_end = (uint32_t)((uint64_t)(part + 1u) * nsteps / parts);
    total = l_end - l_step;
  } else {
    total = (uint64_t)((ntiles - 1u - wg) / grid + 1u) * nsteps;  // grid <= ntiles
  }
  const uint32_t h_tile = l_tile;

  // The step sequence.  One register stage S: during step g (LDS slot g % 2), after
  // the products of its first substep, S (step g + 1, loaded during step g - 1) goes
  // to the other slot and the loads of step g + 2 start into S, so each load has a
  // step of products to arrive.  Whole tiles: the sequence runs across tile
  // boundaries, so the next tile's first steps load while a tile's last step
  // multiplies and its outputs are written.  Every load is issued unconditionally
  // (past the last step, the last tile's or half's last step is re-read), so the
  // only wait for memory is the one before S goes to LDS.
  set_rows(l_tile);
  Stage<T, SCALE_WORDS> S;
  uint32_t s_step = 0;  // K step held in S
  // (selects, no branch, so that the step's products, LDS stores and loads stay in
  // one block the scheduler can interleave)
  auto advance = [&]() {
    if constexpr (SPLIT) {
      l_step = l_step + 1u < l_end ? l_step + 1u : l_step;
    } else {
      const bool wrap = l_step + 1u == nsteps;
      l_step = wrap ? 0u : l_step + 1u;
      l_tile = wrap ? l_tile + grid : l_tile;
      set_rows(l_tile < ntiles ? l_tile : ntiles - 1u);
    }
  };
  auto load_next = [&]() {
    s_step = l_step;
    load_stage(l_step, S);
    advance();
  };
  load_next();
  store_stage(0, s_step, S);
  load_next();
  __syncthreads();
  uint32_t c_tile = wg, c_step = 0;
  for (uint64_t g = 0; g < total; ++g) {
    const int slot = (int)(g & 1u);
    Scales sc;
    read_scales(slot, sc);
    // The stores of S into the other slot go one by one between the first substep's
    // products (the empty asm takes the product just issued, and its memory clobber
    // keeps the store after it), then the loads of the step after next start.
    compute_ks(slot, 0, sc, [&](int u, const v16f& a) {
#if defined(__HIP_DEVICE_COMPILE__)
      asm volatile("" ::"v"(a) : "memory");
#endif
      if (u < T::kChunks) store_chunk(slot ^ 1, u, S);
    });
#pragma unroll
    for (int i = T::kTM * T::kTN; i < T::kChunks; ++i) store_chunk(slot ^ 1, i, S);
    store_scales(slot ^ 1, s_step, S);
    load_next();
#pragma unroll
    for (int ks = 1; ks < kKSub; ++ks) compute_ks(slot, ks, sc, no_hook);
    __syncthreads();
    if constexpr (!SPLIT) {
      if (++c_step == nsteps) {
        if (EPI == kEpiStaged) write_tile_staged(c_tile, slot, NoPartial{});
        else write_tile(c_tile, NoPartial{});
#pragma unroll
        for (int i = 0; i < T::kTM; ++i)
#pragma unroll
          for (int j = 0; j < T::kTN; ++j) acc[i][j] = v16f{};
        c_step = 0;
        c_tile += grid;
      }
    }
  }
  if constexpr (!SPLIT) return;

  // The parts of a split tile meet through its flag word and one fp32 slot of
  // partial sums per part (thread tid's accumulators as 16-byte pieces, piece c at
  // c kThreads + tid; the exchange itself in kq_split.hpp).  The last part adds
  // every part's sums in part order (its own from registers), so the result does
  // not depend on the order of arrival.
  __shared__ uint32_t arrival;
  uint32_t* flag = flags + h_tile;
  // the tile's part slots through one buffer descriptor: piece c of part p's slot
  // for this thread at byte offset 16 tid (per lane) + 16 kThreads c + p x tile
  // bytes (per instruction)
  constexpr int kTileBytes = kBM * T::kBN * 4;
  const __amdgpu_buffer_rsrc_t rsrc_p = __builtin_amdgcn_make_buffer_rsrc(
      partials + (uint64_t)h_tile * parts * (kBM * T::kBN), 0, (int)(parts * (uint32_t)kTileBytes), 0x00020000);
  constexpr int kDeviceCoherent = kSplitCoherent;
  if (!split_arrive_last(flag, parts, arrival)) {
#pragma unroll
    for (int i = 0; i < T::kTM; ++i)
#pragma unroll
      for (int j = 0; j < T::kTN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 v{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rsrc_p, (int)(16u * tid),
                                                 (int)(part * (uint32_t)kTileBytes) +
                                                     16 * kThreads * ((i * T::kTN + j) * 4 + q),
                                                 kDeviceCoherent);
        }
    split_publish(flag);
    return;
  }
  split_wait_reset(flag, parts);
  // The tile's sums, parts 0, 1, ... added in that order (the order of arrival
  // does not matter).  The other parts' slots are loaded branch-free, NO of them
  // per piece, NO = 1, 3 or 7 (the schedule makes it parts - 1; were it more, the
  // loads past the last part would be addressed outside the descriptor's range
  // and return zeros, which add exactly, the sums never being -0 since every
  // accumulation starts at +0).  Other slot k is part k, or k + 1 from this part
  // on.
  auto all_parts_n = [&](auto no_c) {
    constexpr int NO = decltype(no_c)::value;
    return [&](int i, int j, int q, const f32x4& own) {
      const int piece = 16 * kThreads * ((i * T::kTN + j) * 4 + q);
      f32x4 x[NO];
#pragma unroll
      for (int k = 0; k < NO; ++k) {
        const uint32_t pp = (uint32_t)k < part ? (uint32_t)k : (uint32_t)k + 1u;
        // (the whole offset per lane, where the range check applies)
        x[k] = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                       rsrc_p, (int)(16u * tid) + (pp < parts ? (int)pp * kTileBytes + piece : 1 << 30), 0,
                       kDeviceCoherent));
      }
      f32x4 sum = part == 0u ? own : x[0];
#pragma unroll
      for (int pp = 1; pp <= NO; ++pp) {
        // slot pp holds part pp below this part, slot pp - 1 part pp above it (pp = NO
        // is never below: part <= parts - 1 <= NO)
        const f32x4& below = x[pp < NO ? pp : NO - 1];
        sum += (uint32_t)pp == part ? own : (uint32_t)pp < part ? below : x[pp - 1];
      }
      return sum;
    };
  };
  auto write = [&](auto add) {
    if (EPI == kEpiStaged) write_tile_staged(h_tile, 0, add);
    else write_tile(h_tile, add);
  };
  if (parts <= 2u) write(all_parts_n(std::integral_constant<int, 1>{}));
  else if (parts <= 4u) write(all_parts_n(std::integral_constant<int, 3>{}));
  else write(all_parts_n(std::integral_constant<int, kSplitMaxPartsDev - 1>{}));
}

// The static split workspace (kq_mx_gemm_static): zero-initialized with the
// code object; its flags are cleared once more on each device's first use.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

__global__ __launch_bounds__(256) void clear_flags_kernel(uint32_t* __restrict__ flags, uint32_t n) {
  for (uint32_t i = threadIdx.x; i < n; i += blockDim.x) flags[i] = 0u;
}

constexpr int kMaxScratchDevices = 64;
std::once_flag g_scratch_once[kMaxScratchDevices];
void* g_scratch_ptr[kMaxScratchDevices];
hipError_t g_scratch_err[kMaxScratchDevices];

}  // namespace

hipError_t static_scratch(void** ptr, void* stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [&] {
    // the array's device address on this device (in host code its name is only a
    // stand-in); every later use goes through this pointer
    void* p = nullptr;
    hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (r == hipSuccess) {
      hipLaunchKernelGGL(clear_flags_kernel, dim3(1), dim3(256), 0, (hipStream_t)stream,
                         static_cast<uint32_t*>(p), (uint32_t)(kSplitFlagBytes / 4));
      r = hipGetLastError();
    }
    g_scratch_ptr[dev] = r == hipSuccess ? p : nullptr;
    g_scratch_err[dev] = r;
  });
  *ptr = g_scratch_ptr[dev];
  return g_scratch_err[dev];
}

// The grid and the tiles' order for one product (the kernel's unit list).
struct Schedule {
  int64_t tiles_n, ntiles, grid, xcd_cols;
  int64_t band_rows;  // split: tile rows per band of the compact per-XCD order
  bool split;     // every tile in `parts` K parts through the workspace
  int64_t parts;  // K parts per tile (split), workgroup p n8 + t taking part p of tile t
};

// Tiles are split in K only into parts of at least this many K steps (of 256
// values), which make a part worth the exchange of partial sums (two halves
// against the unsplit tile: 4096 x 1152 x 1152, 5 steps: 1.34x the time; 2048 x
// 2240 x 2240, 9 steps: 0.95-1.01x; 256 x 256 x 3072, 12 steps: 0.82-0.85x; 1024
// x 3072 x 12288, 48 steps: 0.70x), and into at most kSplitMaxParts parts.
constexpr int64_t kSplitMinStepsPerPart = 5;
constexpr int64_t kSplitMaxParts = kSplitMaxPartsDev;

// max_slots: the partial-sum tiles the workspace holds (0: whole tiles only).
Schedule make_schedule(int64_t M, int64_t N, int64_t K, int cus, int64_t max_slots) {
  using T = ProductTiling;
  Schedule s{};
  const int64_t tiles_m = (M + T::kBM - 1) / T::kBM;
  s.tiles_n = (N + T::kBN - 1) / T::kBN;
  s.ntiles = tiles_m * s.tiles_n;
  // persistent: at most one workgroup per compute unit (its LDS holds one), a
  // multiple of 8 so that a workgroup's tiles all fall to its XCD's share
  const int64_t full_grid = cus >= 8 ? cus / 8 * 8 : 8;
  const int64_t nsteps = (K + 64 * kKSub - 1) / (64 * kKSub);
  const int64_t n8 = (s.ntiles + 7) / 8 * 8;
  // Splitting pays only while the tiles leave at least half of the compute units
  // idle: with whole rounds of tiles on (nearly) all of them, the matrix cores are
  // power-limited (4608 x 12288 x 3072: the shader clock falls from 1.92 GHz with
  // 216 busy compute units to 1.45-1.69 with 256), so more busy units bring no more
  // throughput, and splitting only adds the exchange.  So: the largest power of
  // two of parts that fits the compute units, with parts of at least
  // kSplitMinStepsPerPart steps, at most kSplitMaxParts, and no more than the
  // workspace holds (one slot per part of every tile).  Powers of two because the
  // last part loads the other parts' slots as 1, 3 or 7 loads per piece, and a
  // count between (a load returning zeros still costs address processing)
  // measured slower: 1024 x 3072 x 12288 in 2, 3, 4 and 5 parts 59.8, 51.5, 48.7
  // and 56.5 us (unsplit 85.1); 512 x 512 x 12288 in 2, 4 and 8 parts 47.2, 38.0
  // and 37.5 us (unsplit 79.3).
  int64_t parts = full_grid / n8;
  parts = parts < nsteps / kSplitMinStepsPerPart ? parts : nsteps / kSplitMinStepsPerPart;
  parts = parts < kSplitMaxParts ? parts : kSplitMaxParts;
  const int64_t fit = s.ntiles > 0 ? max_slots / s.ntiles : 0;
  parts = parts < fit ? parts : fit;
  parts = parts >= 8 ? 8 : parts >= 4 ? 4 : parts >= 2 ? 2 : parts;
  s.split = parts >= 2 && s.ntiles <= kSplitMaxTiles;
  if (s.split) {
    s.parts = parts;
    s.grid = parts * n8;
    // each XCD's tiles, with all their parts, as one compact block (2048 x 3072 x
    // 12288: 67.3-67.8 -> 63.3-63.7 us against row-major tile order)
    s.band_rows = split_band_rows(s.ntiles, s.tiles_n);
  } else {
    // no more workgroups than keep the number of tile rounds, so every workgroup
    // runs the same number of tiles up to one (4608 x 12288: 864 tiles, 216
    // workgroups of 4 instead of 256 of 3 or 4: 121.9 -> 120.1 us)
    s.parts = 1;
    s.grid = full_grid < s.ntiles ? full_grid : s.ntiles;
    const int64_t rounds = (s.ntiles + s.grid - 1) / s.grid;
    int64_t even = (s.ntiles + rounds - 1) / rounds;
    even = (even + 7) / 8 * 8;
    if (even < s.grid) s.grid = even;
  }
  s.xcd_cols = s.tiles_n % 8 == 0 && s.grid % 8 == 0 ? s.tiles_n / 8 : 0;
  return s;
}

int64_t mx_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int cus, int64_t max_slots) {
  const Schedule s = make_schedule(M, N, K, cus, max_slots);
  return s.split ? kSplitFlagBytes + s.parts * s.ntiles * kSplitTileBytes : 0;
}

template <class T, bool OUT_BF16, int EPI, bool SCALE_WORDS, bool SPLIT>
void launch_t(const GemmArgs& g, const Schedule& s) {
  uint8_t* ws = static_cast<uint8_t*>(g.workspace);
  hipLaunchKernelGGL((mx_gemm_kernel<T, OUT_BF16, EPI, SCALE_WORDS, SPLIT>), dim3((unsigned)s.grid),
                     dim3(T::kThreads), 0, (hipStream_t)g.stream, g.qa, (uint32_t)g.lda, g.sa,
                     (uint32_t)g.ldsa, g.qb, (uint32_t)g.ldb, g.sb, (uint32_t)g.ldsb, (uint32_t)g.M,
                     (uint32_t)g.N, (uint32_t)g.K, g.out, (uint32_t)g.ldo, (uint32_t)s.tiles_n,
                     (uint32_t)s.ntiles, (uint32_t)s.xcd_cols, (uint32_t)s.band_rows, (uint32_t)s.parts,
                     reinterpret_cast<uint32_t*>(ws),
                     ws ? reinterpret_cast<float*>(ws + kSplitFlagBytes) : nullptr);
}

template <class T, bool OUT_BF16, int EPI>
void launch_w(const GemmArgs& g, bool words, const Schedule& s) {
  if (s.split) {
    if (words) launch_t<T, OUT_BF16, EPI, true, true>(g, s);
    else launch_t<T, OUT_BF16, EPI, false, true>(g, s);
  } else {
    if (words) launch_t<T, OUT_BF16, EPI, true, false>(g, s);
    else launch_t<T, OUT_BF16, EPI, false, false>(g, s);
  }
}

hipError_t launch_mx_gemm(const GemmArgs& g) {
  using T = ProductTiling;
  // split tiles only as far as the workspace holds their parts
  const int64_t slots = g.workspace != nullptr && g.workspace_bytes >= kSplitFlagBytes
                            ? (g.workspace_bytes - kSplitFlagBytes) / kSplitTileBytes
                            : 0;
  const Schedule s = make_schedule(g.M, g.N, g.K, g.cus, slots);
  // whole 32-bit scale words when every scale row starts 4-byte aligned and holds one
  const bool words = ((uintptr_t)g.sa % 4 == 0) && ((uintptr_t)g.sb % 4 == 0) && g.ldsa % 4 == 0 &&
                     g.ldsb % 4 == 0 && g.K >= 128;
  const int64_t esize = g.out_bf16 ? 2 : 4;
  const bool vec4 = g.N % 4 == 0 && g.ldo % 4 == 0 && (uintptr_t)g.out % (4 * esize) == 0;
  // staged stores address a tile's rows through one buffer descriptor (below 2 GiB)
  const bool staged = g.out_bf16 && g.N % 8 == 0 && g.ldo % 8 == 0 && (uintptr_t)g.out % 16 == 0 &&
                      (int64_t)T::kBM * g.ldo * 2 < (int64_t(1) << 31);
  if (g.out_bf16) {
    if constexpr (T::kCanStage) {
      if (staged) {
        launch_w<T, true, kEpiStaged>(g, words, s);
        return hipGetLastError();
      }
    }
    if (vec4) launch_w<T, true, kEpiVec4>(g, words, s);
    else launch_w<T, true, kEpiScalar>(g, words, s);
  } else {
    if (vec4) launch_w<T, false, kEpiVec4>(g, words, s);
    else launch_w<T, false, kEpiScalar>(g, words, s);
  }
  return hipGetLastError();
}

}  // namespace kq
