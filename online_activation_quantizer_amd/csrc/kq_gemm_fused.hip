// kq_gemm_fused.hip — the W4A4 product with the activation quantizer in its
// prologue (gfx950):
//
//   Y[m][n] = sum_k deq(Q(T X))[m][k] * deq(B)[n][k]
//
// X is the bf16 activation matrix [M][K] and T the per-block transform given by
// its factor parameters (l, u, v) x 5 per 32-channel block (KroQuant researchpod
// summary, method paragraph); Q is the MXFP4 encoding of the quantizer (OCP MX:
// E8M0 scale per 32 values, E2M1 elements).  B is the weights' MXFP4 operand as
// kq_quantize_weights writes it.  KroQuant abstract: the online transform feeds a
// W4A4 MXFP4 product; here its output never leaves the compute unit.
//
// Each workgroup (8 waves, 2 x 4) computes 128 x 256 tiles of Y, each wave a
// 64 x 64 part as 2 x 2 tiles of v_mfma_scale_f32_32x32x64_f8f6f4 (both operands
// fp4, the same instruction, operand layout and K order as kq_mx_gemm).  K advances
// 256 values per step.  Per step, every thread quantizes two (row, block) units of
// the activation tile: it loads the unit's 32 bf16 values, applies the block's
// transform and encodes it with the quantizer's own device functions (so the codes
// and scales equal kq_quantize's bit for bit) and writes the 16 code bytes and the
// scale byte into LDS where the matrix cores read them; the weight tile's codes and
// scales are copied to LDS beside them.  Every block's 42 transform constants are
// built once per workgroup into LDS (K <= 16384).  The activation tile is quantized
// again for every tile column of Y, so this path pays where Y has few tile columns;
// with many, quantizing once (kq_quantize) and reading the 4.25x smaller MXFP4
// operand is cheaper.
//
// Split tiles (kq_mx_gemm_fused_ws, kernel variant SPLIT).  With few tiles most
// compute units idle, and each tile's quantization is the bulk of its work: each
// tile is computed as S parts of K on S workgroups of its XCD, each quantizing and
// multiplying only its K steps (and building only its blocks' constants); the parts
// meet through a workspace as the W4A4 product's split tiles do (kq_split.hpp), the
// last adding every part's sums in part order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kq_device.hpp"
#include "kq_factors.hpp"
#include "kq_launch.hpp"
#include "kq_split.hpp"

// Products and sums round separately unless written as an explicit fma.
#pragma clang fp contract(off)

namespace kq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kFThreads = 512;
constexpr int kFBM = 128, kFBN = 256;        // output tile
constexpr int kFRows = kFBM + kFBN;          // LDS code rows: the activations', then the weights'
constexpr int kFStepBytes = 128;             // code bytes per row per K step (256 values)
constexpr int kFPitch = kFStepBytes + 16;    // LDS code-row pitch (bank spread)
constexpr int kFConstStride = 44;            // floats per block's constants in LDS
constexpr int kFUnits = kFBM * 8 / kFThreads;              // activation units per thread per step
constexpr int kFChunks = kFBN * (kFStepBytes / 16) / kFThreads;  // weight code chunks per thread

template <bool OUT_BF16, bool VEC4, bool SPLIT>
__global__ __launch_bounds__(kFThreads) __attribute__((amdgpu_waves_per_eu(2))) void fused_gemm_kernel(
    const uint8_t* __restrict__ x, uint32_t ldx, const float* __restrict__ params,
    const uint8_t* __restrict__ qb, uint32_t ldb, const uint8_t* __restrict__ sb, uint32_t ldsb,
    uint32_t M, uint32_t N, uint32_t K, void* __restrict__ out, uint32_t ldo, uint32_t tiles_n,
    uint32_t ntiles, uint32_t band_rows, uint32_t parts, uint32_t* __restrict__ flags,
    float* __restrict__ partials) {
  __shared__ __attribute__((aligned(16))) uint8_t codes[kFRows * kFPitch];
  __shared__ __attribute__((aligned(16))) uint8_t scale_bytes[kFRows * 8];  // 8 per row per step
  __shared__ __attribute__((aligned(16))) float consts[kFusedMaxBlocks * kFConstStride];
  const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
  const uint32_t wm = wave / 4u, wn = wave % 4u;
  const uint32_t lr = lane & 31u, h = lane >> 5;
  const uint32_t kblocks = K / 32u, kbytes = K / 2u;
  const uint32_t nsteps = (K + 255u) / 256u;

  // This workgroup's tiles t_begin, + t_stride, ... and K steps [step_lo,
  // step_hi).  SPLIT: one K part of one tile, workgroup p n8 + t (n8 = ntiles
  // rounded up to 8, so all parts of a tile run on its XCD) taking steps
  // [p nsteps / parts, (p + 1) nsteps / parts) of tile t.
  uint32_t t_begin = blockIdx.x, t_stride = gridDim.x, step_lo = 0, step_hi = nsteps;
  [[maybe_unused]] uint32_t part = 0;
  if constexpr (SPLIT) {
    const uint32_t n8 = (ntiles + 7u) & ~7u;
    part = blockIdx.x / n8;
    t_begin = blockIdx.x - part * n8;
    if (t_begin >= ntiles || part >= parts) return;
    t_stride = ntiles;  // one tile
    step_lo = (uint32_t)((uint64_t)part * nsteps / parts);
    step_hi = (uint32_t)((uint64_t)(part + 1u) * nsteps / parts);
  }
  const uint32_t b_lo = step_lo * 8u, b_hi = step_hi * 8u < kblocks ? step_hi * 8u : kblocks;

  // The constants (the diagonal, then the upper and lower shear coefficients) of
  // every block of the workgroup's K steps, once per workgroup.
  for (uint32_t b = b_lo + tid; b < b_hi; b += kFThreads) {
    BlockParams bp;
#pragma unroll
    for (int i = 0; i < 15; ++i) bp.p[i] = params[(size_t)b * 15 + i];
    BlockConsts c;
    make_consts<false>(bp, c);
    float* dst = consts + b * kFConstStride;
#pragma unroll
    for (int i = 0; i < kBlk; ++i) dst[i] = c.d[i];
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      dst[kBlk + k] = c.su[k];
      dst[kBlk + 5 + k] = c.ll[k];
    }
  }
  __syncthreads();
  auto read_consts = [&](uint32_t b, BlockConsts& c) {
    const f32x4* src = reinterpret_cast<const f32x4*>(consts + b * kFConstStride);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const f32x4 v = src[k];
      c.d[4 * k] = v.x;
      c.d[4 * k + 1] = v.y;
      c.d[4 * k + 2] = v.z;
      c.d[4 * k + 3] = v.w;
    }
    const f32x4 a = src[8], bq = src[9], cq = src[10];
    const float rest[12] = {a.x, a.y, a.z, a.w, bq.x, bq.y, bq.z, bq.w, cq.x, cq.y, cq.z, cq.w};
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      c.su[k] = rest[k];
      c.ll[k] = rest[5 + k];
    }
  };

  for (uint32_t t = t_begin; t < ntiles; t += t_stride) {
    // (split: each XCD's tiles as one compact block of the tile grid, split_tile)
    uint32_t tm = t / tiles_n, tn = t - tm * tiles_n;
    if constexpr (SPLIT) split_tile(t, ntiles, tiles_n, band_rows, tm, tn);
    const uint32_t m0 = tm * kFBM, n0 = tn * kFBN;
    v16f acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};

    for (uint32_t step = step_lo; step < step_hi; ++step) {
      // Loads of this step, all issued before any arithmetic waits on them.
      // Activation unit i of this thread: row r = u / 8 of the tile, block j = u % 8
      // of the step (u = tid + 512 i; consecutive threads read consecutive 64-byte
      // blocks of a row).  Rows past M re-read the last row (not stored); blocks past
      // K re-read the last block and are encoded as zero codes with scale 0x00.
      // (Issuing the next step's loads before this step's products measured slower:
      // 53.0 -> 59.9 us at 4608 x 256 x 3072.)
      Raw<DT_BF16> raw[kFUnits];
#pragma unroll
      for (int i = 0; i < kFUnits; ++i) {
        const uint32_t u = tid + kFThreads * i, r = u / 8u, j = u % 8u;
        const uint32_t row = m0 + r < M ? m0 + r : M - 1u;
        const uint32_t kb = step * 8u + j < kblocks ? step * 8u + j : kblocks - 1u;
        raw[i] = load_raw<DT_BF16>(x + (uint64_t)row * ldx + (uint64_t)kb * (kBlk * 2));
      }
      // Weight code chunk i: row c / 8 of the tile, 16-byte column c % 8 of the step
      // (c = tid + 512 i); past K the row's last chunk (its scale becomes 0x00).
      u32x4 wc[kFChunks];
#pragma unroll
      for (int i = 0; i < kFChunks; ++i) {
        const uint32_t c = tid + kFThreads * i, r = c / 8u, col = 16u * (c % 8u);
        const uint32_t row = n0 + r < N ? n0 + r : N - 1u;
        const uint32_t at = step * kFStepBytes + col < kbytes ? step * kFStepBytes + col : kbytes - 16u;
        wc[i] = *reinterpret_cast<const u32x4*>(qb + (uint64_t)row * ldb + at);
      }
      // Weight scale bytes: thread tid < 256 takes row tid's 8 of this step.
      uint32_t ws[8];
      {
        const uint32_t r = tid < (uint32_t)kFBN ? tid : kFBN - 1u;
        const uint32_t row = n0 + r < N ? n0 + r : N - 1u;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const uint32_t kb = step * 8u + q < kblocks ? step * 8u + q : kblocks - 1u;
          ws[q] = sb[(uint64_t)row * ldsb + kb];
        }
      }

      // Quantize the activation units into LDS (the quantizer's transform and encoder).
#pragma unroll
      for (int i = 0; i < kFUnits; ++i) {
        const uint32_t u = tid + kFThreads * i, r = u / 8u, j = u % 8u;
        const uint32_t kb = step * 8u + j;
        float v[kBlk];
        unpack(raw[i], v);
        BlockConsts c;
        read_consts(kb < kblocks ? kb : kblocks - 1u, c);
        transform<false>(v, c);
        uint32_t w[4];
        const uint32_t S = encode(v, w);
        const bool in_k = kb < kblocks;
        *reinterpret_cast<u32x4*>(&codes[r * kFPitch + 16u * j]) =
            in_k ? u32x4{w[0], w[1], w[2], w[3]} : u32x4{0u, 0u, 0u, 0u};
        scale_bytes[r * 8u + j] = in_k ? (uint8_t)S : (uint8_t)0u;
      }
#pragma unroll
      for (int i = 0; i < kFChunks; ++i) {
        const uint32_t c = tid + kFThreads * i;
        *reinterpret_cast<u32x4*>(&codes[(kFBM + c / 8u) * kFPitch + 16u * (c % 8u)]) = wc[i];
      }
      if (tid < (uint32_t)kFBN) {
#pragma unroll
        for (int q = 0; q < 8; ++q)
          scale_bytes[(kFBM + tid) * 8u + q] = step * 8u + q < kblocks ? (uint8_t)ws[q] : (uint8_t)0u;
      }
      __syncthreads();

      // The products: the wave's activation row tiles i and weight row tiles j.
      uint32_t sa[2][2], sbw[2][2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t ra = wm * 64u + 32u * i + lr, rb = kFBM + wn * 64u + 32u * i + lr;
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          sa[i][w] = reinterpret_cast<const uint32_t*>(scale_bytes)[ra * 2u + w];
          sbw[i][w] = reinterpret_cast<const uint32_t*>(scale_bytes)[rb * 2u + w];
        }
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        v8i A[2], B[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const uint32_t ra = wm * 64u + 32u * i + lr, rb = kFBM + wn * 64u + 32u * i + lr;
          const u32x4 va = *reinterpret_cast<const u32x4*>(&codes[ra * kFPitch + 32u * ks + 16u * h]);
          const u32x4 vb = *reinterpret_cast<const u32x4*>(&codes[rb * kFPitch + 32u * ks + 16u * h]);
          A[i] = v8i{(int)va.x, (int)va.y, (int)va.z, (int)va.w, 0, 0, 0, 0};
          B[i] = v8i{(int)vb.x, (int)vb.y, (int)vb.z, (int)vb.w, 0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            // the lane's block scale (byte 2 ks + h of the row's step) moved to byte
            // 2 (ks % 2) of its word, which op_sel picks; the weights are the first operand
            const int sA = (int)(sa[i][ks / 2] >> (8u * h)), sB = (int)(sbw[j][ks / 2] >> (8u * h));
            if (ks % 2 == 0)
              acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(B[j], A[i], acc[i][j], 4, 4, 0, sB, 0, sA);
            else
              acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(B[j], A[i], acc[i][j], 4, 4, 2, sB, 2, sA);
          }
      }
      __syncthreads();
    }

    // acc[i][j][4 q + e]: Y row lr of the wave's activation tile i, column
    // 8 q + 4 h + e of its weight tile j.  `sums(i, j, own, sv)` turns the four
    // pieces own[q] = acc[i][j][4 q .. 4 q + 3] into their outputs sv[q]: their own
    // values, or the whole split tile's.
    auto write_tile = [&](auto sums) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t row = m0 + wm * 64u + 32u * i + lr;
        if (row >= M) continue;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          f32x4 own[4], sv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            own[q] = f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          sums(i, j, own, sv);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t col = n0 + wn * 64u + 32u * j + 8u * q + 4u * h;
            const float v[4] = {sv[q].x, sv[q].y, sv[q].z, sv[q].w};
            if (OUT_BF16) {
              uint32_t bw[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                // round to nearest even (finite values)
                const uint32_t uu = __float_as_uint(v[e]);
                bw[e] = (uu + 0x7FFFu + ((uu >> 16) & 1u)) >> 16;
              }
              uint16_t* p = reinterpret_cast<uint16_t*>(out) + (uint64_t)row * ldo + col;
              if (VEC4) {
                if (col < N) *reinterpret_cast<u32x2*>(p) = u32x2{bw[0] | (bw[1] << 16), bw[2] | (bw[3] << 16)};
              } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  if (col + e < N) p[e] = (uint16_t)bw[e];
              }
            } else {
              float* p = reinterpret_cast<float*>(out) + (uint64_t)row * ldo + col;
              if (VEC4) {
                if (col < N) *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
              } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  if (col + e < N) p[e] = v[e];
              }
            }
          }
        }
      }
    };
    if constexpr (!SPLIT) {
      write_tile([](int, int, const f32x4 (&own)[4], f32x4 (&sv)[4]) {
#pragma unroll
        for (int q = 0; q < 4; ++q) sv[q] = own[q];
      });
    } else {
      // The parts meet through the tile's flag word and one fp32 slot of partial
      // sums per part (thread tid's accumulators as 16-byte pieces, piece c at
      // c kFThreads + tid), as kq_split.hpp describes.
      __shared__ uint32_t arrival;
      uint32_t* flag = flags + t;
      constexpr int kTileBytes = kFBM * kFBN * 4;
      const __amdgpu_buffer_rsrc_t rsrc_p = __builtin_amdgcn_make_buffer_rsrc(
          partials + (uint64_t)t * parts * (kFBM * kFBN), 0, (int)(parts * (uint32_t)kTileBytes), 0x00020000);
      if (!split_arrive_last(flag, parts, arrival)) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const f32x4 v{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
              __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rsrc_p, (int)(16u * tid),
                                                     (int)(part * (uint32_t)kTileBytes) +
                                                         16 * kFThreads * ((i * 2 + j) * 4 + q),
                                                     kSplitCoherent);
            }
        split_publish(flag);
        return;
      }
      split_wait_reset(flag, parts);
      // (the part numbers pass through an empty asm here, so that the slot offsets
      // computed from them are not hoisted above the K loop, where they would hold
      // registers the loop needs)
      uint32_t my_part = part, n_parts = parts;
      asm volatile("" : "+s"(my_part), "+s"(n_parts));
      // every part's sums in part order: the other parts' slots as NO branch-free
      // loads per piece (NO = parts - 1 = 1, 3 or 7; other slot k is part k, or
      // k + 1 from this part on), this part's from registers; the four pieces of
      // one 32 x 32 tile at a time (all of them in flight at once would not fit
      // the registers)
      auto all_parts_n = [&](auto no_c) {
        constexpr int NO = decltype(no_c)::value;
        return [&](int i, int j, const f32x4 (&own)[4], f32x4 (&sv)[4]) {
          f32x4 xs[4][NO];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int piece = 16 * kFThreads * ((i * 2 + j) * 4 + q);
#pragma unroll
            for (int k = 0; k < NO; ++k) {
              const uint32_t pp = (uint32_t)k < my_part ? (uint32_t)k : (uint32_t)k + 1u;
              // (the whole offset per lane, where the range check applies: a slot past
              // the last part reads zeros, which add exactly)
              xs[q][k] = __builtin_bit_cast(
                  f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                             rsrc_p, (int)(16u * tid) + (pp < n_parts ? (int)pp * kTileBytes + piece : 1 << 30), 0,
                             kSplitCoherent));
            }
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            f32x4 sum = my_part == 0u ? own[q] : xs[q][0];
#pragma unroll
            for (int pp = 1; pp <= NO; ++pp) {
              const f32x4& below = xs[q][pp < NO ? pp : NO - 1];
              sum += (uint32_t)pp == my_part ? own[q] : (uint32_t)pp < my_part ? below : xs[q][pp - 1];
            }
            sv[q] = sum;
          }
          __builtin_amdgcn_sched_barrier(0);
        };
      };
      if (n_parts <= 2u) write_tile(all_parts_n(std::integral_constant<int, 1>{}));
      else if (n_parts <= 4u) write_tile(all_parts_n(std::integral_constant<int, 3>{}));
      else write_tile(all_parts_n(std::integral_constant<int, 7>{}));
    }
  }
}

// The fused product's schedule: whole tiles on a persistent grid (one workgroup per
// compute unit), or, with a workspace and few tiles, every tile in S parts of K.
// Its parts are shorter than the W4A4 product's (kFusedMinStepsPerPart steps),
// each step holding the quantization of a tile's worth of activations.
constexpr int64_t kFusedMinStepsPerPart = 3;
struct FusedSchedule {
  int64_t tiles_n, ntiles, grid, parts;
  int64_t band_rows;  // split: tile rows per band of the compact per-XCD order
  bool split;
};

FusedSchedule fused_schedule(int64_t M, int64_t N, int64_t K, int cus, int64_t max_slots) {
  FusedSchedule s{};
  const int64_t tiles_m = (M + kFBM - 1) / kFBM;
  s.tiles_n = (N + kFBN - 1) / kFBN;
  s.ntiles = tiles_m * s.tiles_n;
  const int64_t full_grid = cus >= 8 ? cus / 8 * 8 : 8;
  const int64_t nsteps = (K + 255) / 256;
  const int64_t n8 = (s.ntiles + 7) / 8 * 8;
  // the largest of 2, 4 and 8 parts that fits the compute units, with parts of at
  // least kFusedMinStepsPerPart steps, and no more than the workspace holds
  int64_t parts = full_grid / n8;
  parts = parts < nsteps / kFusedMinStepsPerPart ? parts : nsteps / kFusedMinStepsPerPart;
  const int64_t fit = s.ntiles > 0 ? max_slots / s.ntiles : 0;
  parts = parts < fit ? parts : fit;
  parts = parts >= 8 ? 8 : parts >= 4 ? 4 : parts >= 2 ? 2 : parts;
  s.split = parts >= 2 && s.ntiles <= kSplitMaxTiles;
  s.parts = s.split ? parts : 1;
  s.grid = s.split ? parts * n8 : (s.ntiles < cus ? s.ntiles : cus);
  s.band_rows = s.split ? split_band_rows(s.ntiles, s.tiles_n) : 1;
  return s;
}

template <bool OUT_BF16, bool VEC4, bool SPLIT>
void launch_fused_t(const FusedGemmArgs& g, const FusedSchedule& s) {
  uint8_t* ws = static_cast<uint8_t*>(g.workspace);
  hipLaunchKernelGGL((fused_gemm_kernel<OUT_BF16, VEC4, SPLIT>), dim3((unsigned)s.grid), dim3(kFThreads), 0,
                     (hipStream_t)g.stream, static_cast<const uint8_t*>(g.x), (uint32_t)(g.ldx * 2),
                     g.params, g.qb, (uint32_t)g.ldb, g.sb, (uint32_t)g.ldsb, (uint32_t)g.M,
                     (uint32_t)g.N, (uint32_t)g.K, g.out, (uint32_t)g.ldo, (uint32_t)s.tiles_n,
                     (uint32_t)s.ntiles, (uint32_t)s.band_rows, (uint32_t)s.parts, reinterpret_cast<uint32_t*>(ws),
                     ws ? reinterpret_cast<float*>(ws + kSplitFlagBytes) : nullptr);
}

template <bool OUT_BF16, bool VEC4>
void launch_fused_s(const FusedGemmArgs& g, const FusedSchedule& s) {
  if (s.split) launch_fused_t<OUT_BF16, VEC4, true>(g, s);
  else launch_fused_t<OUT_BF16, VEC4, false>(g, s);
}

}  // namespace

int64_t mx_gemm_fused_workspace_bytes(int64_t M, int64_t N, int64_t K, int cus) {
  const FusedSchedule s = fused_schedule(M, N, K, cus, INT64_MAX);
  return s.split ? kSplitFlagBytes + s.parts * s.ntiles * kFusedSplitTileBytes : 0;
}

hipError_t launch_mx_gemm_fused(const FusedGemmArgs& g) {
  // split tiles only as far as the workspace holds their parts
  const int64_t slots = g.workspace != nullptr && g.workspace_bytes >= kSplitFlagBytes
                            ? (g.workspace_bytes - kSplitFlagBytes) / kFusedSplitTileBytes
                            : 0;
  const FusedSchedule s = fused_schedule(g.M, g.N, g.K, g.cus, slots);
  const int64_t esize = g.out_bf16 ? 2 : 4;
  const bool vec4 = g.N % 4 == 0 && g.ldo % 4 == 0 && (uintptr_t)g.out % (4 * esize) == 0;
  if (g.out_bf16) {
    if (vec4) launch_fused_s<true, true>(g, s);
    else launch_fused_s<true, false>(g, s);
  } else {
    if (vec4) launch_fused_s<false, true>(g, s);
    else launch_fused_s<false, false>(g, s);
  }
  return hipGetLastError();
}

}  // namespace kq
