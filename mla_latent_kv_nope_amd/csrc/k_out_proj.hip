// mla_out_proj: out[b][h] = W_UV[h]^T . o_lat[b][h].
//
// Method: W_UV is absorbed into the output side ("DeepSeek-V2拆解：MLA与MoE如何把
// KV缓存压降93.3%", sheratonhq.com, section 2.1), so the attention result stays
// in the d_c-wide latent space until this per-head projection.
//
// A per-head batched GEMM [B x d_c] x [d_c x d_v] on 32x32x16 bf16 MFMA.  One
// wave computes a 32 x 32 output tile (32 batch rows x 32 columns of one head).
// The o_lat operand is contiguous along the reduction axis and goes straight
// into MFMA registers.  W_UV[h] is stored [d_c][d_v] (contiguous along the
// output axis), so the wave's [d_c x 32] slice is copied to LDS and read back
// with the gfx950 transpose read, which hands each lane four consecutive
// reduction elements of its output column.  Every global load of a wave is in
// flight at once: the kernel is a single memory round trip per wave.
#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {
namespace {

template <int DC, int DV>
__global__ __launch_bounds__(64) void k_out_proj(OutProjArgs a) {
  constexpr int NCOL = 32;                      // output columns per wave (MFMA N)
  constexpr int KC = DC / 16;                   // reduction chunks
  static_assert(DC % 16 == 0 && (DC * NCOL) % 512 == 0, "tile shape");
  // [DC][32] bf16 slice, row-major; 16 consecutive lanes of a transpose read
  // touch 4 rows x 32 bytes, which fall in distinct banks
  __shared__ __attribute__((aligned(1024))) uint16_t w[DC * NCOL];

  const int h = blockIdx.x;
  const int v0 = blockIdx.y * NCOL;
  const int b0 = blockIdx.z * 32;
  const int lane = threadIdx.x;
  const int B = a.B, H = a.H;

  // stage W_UV[h][:, v0:v0+32].  With whole 32-column slices, 16-byte
  // global->LDS copies: lane l of copy k moves elements [8(l%4), +8) of row
  // 16k + l/4, which is exactly LDS byte 1024k + 16l of the row-major slice.
  const uint16_t* wsrc = a.w_uv + static_cast<int64_t>(h) * DC * DV;
  if constexpr (DV % NCOL == 0) {
#pragma unroll
    for (int k = 0; k < DC * NCOL / 512; ++k) {
      const int i = k * 64 + lane;
      const uint16_t* src = wsrc + (i >> 2) * DV + v0 + (i & 3) * 8;
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const void*>(src),
          reinterpret_cast<lds_void_t*>(reinterpret_cast<uintptr_t>(w) + 1024 * k), 16, 0, 0);
    }
  } else {
    for (int i = lane; i < DC * (NCOL / 8); i += 64) {
      const int r = i >> 2, c8 = (i & 3) * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (v0 + c8 < DV) v = *reinterpret_cast<const uint4*>(wsrc + r * DV + v0 + c8);
      *reinterpret_cast<uint4*>(&w[r * NCOL + c8]) = v;
    }
  }

  // o_lat rows b0 + lane%32, all loads in flight together with the copies
  const int half = lane >> 5;
  const int br = b0 + (lane & 31);
  const bool ok = br < B;
  const uint16_t* orow = a.o_lat + (static_cast<int64_t>(ok ? br : 0) * H + h) * DC + 8 * half;
  bf16x8 av[KC];
  const bf16x8 z = {};
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(orow + 16 * k);
    av[k] = ok ? v : z;
  }
  wait_vmcnt<0>();
  __syncthreads();

  // transpose-read addressing: source lane 4r+q of its 16-lane group reads
  // reduction row (8*g + r [+4]) at columns [16*(G%2) + 4q, +4) of this slice
  const int G = lane >> 4, j = lane & 15, rr = j >> 2, q = j & 3, g = lane >> 5;
  const int col0 = 16 * (G & 1) + 4 * q;
  f32x16 acc = {};
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    const int row = 16 * k + 8 * g + rr;
    const bf16x4 lo = lds_read_tr16(&w[row * NCOL + col0]);
    const bf16x4 hi = lds_read_tr16(&w[(row + 4) * NCOL + col0]);
    const bf16x8 bv = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    acc = mfma32(av[k], bv, acc);
  }
  const int c = v0 + (lane & 31);
  if (c < DV) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int b = b0 + 8 * (i >> 2) + 4 * half + (i & 3);
      if (b < B) a.out[(static_cast<int64_t>(b) * H + h) * DV + c] = f32_to_bf16_bits(acc[i]);
    }
  }
}

// d_c 512, d_v 128: one workgroup of four waves per (head h, 64 output
// columns, 64 batch rows); wave w computes the 32 x 32 tile (rows 32 (w & 1),
// columns 32 (w >> 1)).  The W_UV slice [512][64] (128-byte rows, whole cache
// lines) and the 64 o_lat rows (1 KB each) are copied global->LDS, so each
// byte leaves L2 once per workgroup (half the traffic of one wave per 32 x 32
// tile, which re-read o_lat rows for every column tile).  LDS layouts (16-byte
// chunks permuted within a row, so every copy still reads whole lines):
//   W slice: chunk c of row k at c ^ 2 (k mod 4), so the 4 rows x 32 bytes a
//            transpose read's 16-lane group touches fall in distinct banks;
//   o_lat:   chunk j of row r at j ^ (r mod 32), so the 32 rows an A-operand
//            read touches at one column spread over the banks.
__global__ __launch_bounds__(256) void k_out_proj_w(OutProjArgs a) {
  constexpr int DC = 512, DV = 128, NC = 64, MR = 64;     // columns, rows per workgroup
  constexpr int WROW = NC * 2;                            // bytes per W slice row
  __shared__ __attribute__((aligned(1024))) char wl[DC * WROW];   // 64 KB
  __shared__ __attribute__((aligned(1024))) char ol[MR * DC * 2]; // 64 KB
  const int h = blockIdx.x;
  const int n0 = blockIdx.y * NC;
  const int b0 = blockIdx.z * MR;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int B = a.B, H = a.H;

  // W slice: copy k covers rows 8k .. 8k + 7; lane l fills row 8k + l/8 at
  // chunk position l % 8 with logical chunk (l % 8) ^ 2 (row mod 4)
  const uint16_t* wsrc = a.w_uv + static_cast<int64_t>(h) * DC * DV + n0;
  for (int k = wave; k < DC / 8; k += 4) {
    const int r = 8 * k + (lane >> 3);
    const int c = (lane & 7) ^ (2 * (r & 3));
    lds_dma16_v(wsrc + r * DV + 8 * c, lds_addr(wl + 1024 * k));
  }
  // o_lat rows: copy r is row b0 + r; lane l fills chunk position l with
  // logical chunk l ^ (r mod 32); rows past the batch copy row b0
  for (int r = wave; r < MR; r += 4) {
    const int br = b0 + r < B ? b0 + r : b0;
    const int c = lane ^ (r & 31);
    lds_dma16_v(a.o_lat + (static_cast<int64_t>(br) * H + h) * DC + 8 * c, lds_addr(ol + 1024 * r));
  }
  wait_vmcnt<0>();
  __syncthreads();

  const int rt = wave & 1, ct = wave >> 1;
  // A: row 32 rt + l%32, k = 16 s + 8 (l/32) + [0, 8): logical chunk 2 s + l/32
  const int ar = 32 * rt + (lane & 31), ah = lane >> 5;
  const char* arow = ol + ar * (DC * 2);
  // B (transpose reads): source lane 4 rr + q of 16-lane group G reads row
  // 16 s + 8 (l/32) + rr (+4 for the upper half), columns col0 .. col0 + 3
  const int G = lane >> 4, j = lane & 15, rr = j >> 2, q = j & 3, g = lane >> 5;
  const int col0 = 32 * ct + 16 * (G & 1) + 4 * q;       // column within the slice
  f32x16 acc = {};
#pragma unroll 8
  for (int s = 0; s < DC / 16; ++s) {
    const bf16x8 av = *reinterpret_cast<const bf16x8*>(arow + 16 * ((2 * s + ah) ^ (ar & 31)));
    const int row = 16 * s + 8 * g + rr;                   // row % 4 == rr
    const int cb = ((col0 >> 3) ^ (2 * rr)) * 16 + (col0 & 7) * 2;   // byte offset in the row
    const bf16x4 lo = lds_read_tr16(wl + row * WROW + cb);
    const bf16x4 hi = lds_read_tr16(wl + (row + 4) * WROW + cb);
    const bf16x8 bv = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    acc = mfma32(av, bv, acc);
  }
  // acc[i]: row 32 rt + 8 (i/4) + 4 (l/32) + i%4, column 32 ct + l%32
  const int c = n0 + 32 * ct + (lane & 31);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int b = b0 + 32 * rt + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
    if (b < B) a.out[(static_cast<int64_t>(b) * H + h) * DV + c] = f32_to_bf16_bits(acc[i]);
  }
}

}  // namespace

bool out_proj_supported(int d_c, int d_v) {
  return (d_c == 512 && d_v == 128) || (d_c == 32 && d_v == 16);
}

hipError_t launch_out_proj(const OutProjArgs& a, hipStream_t s) {
  if (a.d_c == 512 && a.d_v == 128) {
    hipLaunchKernelGGL(k_out_proj_w, dim3(a.H, 128 / 64, (a.B + 63) / 64), dim3(256), 0, s, a);
  } else if (a.d_c == 32 && a.d_v == 16) {
    hipLaunchKernelGGL((k_out_proj<32, 16>), dim3(a.H, 1, (a.B + 31) / 32), dim3(64), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla
