// Repack canonical block bytes into the tile-block layout the GEMM streams
// (layout documented in sv_internal.h).  One thread per (output row,
// super-block); every write of a thread lands in its own column's slots, so
// threads never overlap.  A row map lets one repack fuse several canonical
// tensors (q|k|v, interleaved gate/up) and permute rows (RoPE pairs).
#include "sv_device.h"
#include "sv_internal.h"

__device__ __forceinline__ uint32_t slot_bit(int s) { return 4 * (s >> 1) + 16 * (s & 1); }

__device__ __forceinline__ int nib(const uint8_t *p, int k) { return (p[k >> 1] >> (4 * (k & 1))) & 15; }

// 8 codes of k-octet (ks, g) packed in slot order.
__device__ __forceinline__ uint32_t pack_octet(const int *q, int ks, int g) {
  uint32_t w = 0;
  for (int s = 0; s < 8; ++s) w |= (uint32_t)(q[32 * ks + 8 * g + s] & 15) << slot_bit(s);
  return w;
}

__global__ void k_repack(int type, const uint8_t *const *srcs, const int32_t *rowmap,
                         int64_t nrows, int nsb, uint8_t *dst) {
  int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= nrows * nsb) return;
  int64_t n = tid / nsb;
  int sb = (int)(tid % nsb);
  int32_t rm = rowmap[n];
  const uint8_t *src = srcs[rm >> 24];
  int64_t srow = rm & 0xFFFFFF;
  int c = (int)(n & 15);
  int q[256];
  if (type == SV_B6_256) {
    const uint8_t *b = src + (srow * nsb + sb) * 210;
    uint8_t *tb = dst + ((n >> 4) * nsb + sb) * (int64_t)SV_TB_B6;
    for (int j = 0; j < 16; ++j) tb[16 * c + j] = b[192 + j];
    tb[256 + 2 * c] = b[208];
    tb[256 + 2 * c + 1] = b[209];
    for (int k = 0; k < 256; ++k)
      q[k] = nib(b, k) | (((b[128 + (k >> 2)] >> (2 * (k & 3))) & 3) << 4);
    for (int ks = 0; ks < 8; ++ks)
      for (int g = 0; g < 4; ++g) {
        uint32_t *lo = (uint32_t *)(tb + 288 + 1024 * (ks >> 2) + 16 * (c + 16 * g) + 4 * (ks & 3));
        *lo = pack_octet(q, ks, g);
      }
    for (int i = 0; i < 4; ++i)
      for (int g = 0; g < 4; ++g) {
        uint32_t w = 0;
        for (int a = 0; a < 2; ++a) {
          int ks = 2 * i + a;
          for (int s = 0; s < 8; ++s) {
            int hi = (q[32 * ks + 8 * g + s] >> 4) & 3;
            w |= (uint32_t)hi << (8 * a + 2 * (s >> 1) + 16 * (s & 1));
          }
        }
        *(uint32_t *)(tb + 2336 + 16 * (c + 16 * g) + 4 * i) = w;
      }
    return;
  }
  uint8_t *tb = dst + ((n >> 4) * nsb + sb) * (int64_t)SV_TB_B4;
  if (type == SV_B4_256) {
    const uint8_t *b = src + (srow * nsb + sb) * 144;
    int f[16];
    for (int i = 0; i < 16; ++i) {
      int v = 0;
      for (int bit = 0; bit < 6; ++bit) {
        int pos = 6 * i + bit;
        v |= ((b[4 + (pos >> 3)] >> (pos & 7)) & 1) << bit;
      }
      f[i] = v;
    }
    // record: dword0 d | dmin << 16; dwords 1 and 2 hold sc_{4h..4h+3} and
    // the high bits of m_{4h..4h+3} (h = 0, 1); dword 3 the low nibbles of m.
    // Positions are chosen so that pairs come out with one shift and mask:
    //   sc pair (4h, 4h+1) = dw & 0x003F003F, (4h+2, 4h+3) = (dw >> 6) & ...;
    //   m low pair (2i, 2i+1) = (dw3 >> 4i) & 0x000F000F;
    //   m high pair (4h, 4h+1) = (dw >> 12) & 0x00030003, (4h+2, 4h+3) >> 14.
    uint8_t *rec = tb + 16 * c;
    rec[0] = b[0]; rec[1] = b[1]; rec[2] = b[2]; rec[3] = b[3];
    for (int h = 0; h < 2; ++h) {
      const int *sc = f + 4 * h, *mm = f + 8 + 4 * h;
      uint32_t dw = (uint32_t)sc[0] | ((uint32_t)sc[2] << 6) | ((uint32_t)(mm[0] >> 4) << 12) |
                    ((uint32_t)(mm[2] >> 4) << 14) | ((uint32_t)sc[1] << 16) |
                    ((uint32_t)sc[3] << 22) | ((uint32_t)(mm[1] >> 4) << 28) |
                    ((uint32_t)(mm[3] >> 4) << 30);
      *(uint32_t *)(rec + 4 + 4 * h) = dw;
    }
    uint32_t d3 = 0;
    for (int i = 0; i < 4; ++i)
      d3 |= ((uint32_t)(f[8 + 2 * i] & 15) << (4 * i)) |
            ((uint32_t)(f[8 + 2 * i + 1] & 15) << (16 + 4 * i));
    *(uint32_t *)(rec + 12) = d3;
    for (int k = 0; k < 256; ++k) q[k] = nib(b + 16, k);
  } else {  // SV_B4_32: the super-block is 8 consecutive 32-blocks
    const uint8_t *b = src + (srow * nsb + sb) * 144;
    uint8_t *rec = tb + 16 * c;
    for (int j = 0; j < 8; ++j) {
      const uint8_t *blk = b + 18 * j;
      rec[2 * j] = blk[0];
      rec[2 * j + 1] = blk[1];
      for (int t = 0; t < 32; ++t) q[32 * j + t] = nib(blk + 2, t);
    }
  }
  for (int ks = 0; ks < 8; ++ks)
    for (int g = 0; g < 4; ++g)
      *(uint32_t *)(tb + 256 + 1024 * (ks >> 2) + 16 * (c + 16 * g) + 4 * (ks & 3)) =
          pack_octet(q, ks, g);
}

hipError_t sv_launch_repack(int type, const uint8_t *const *srcs_dev, const int32_t *rowmap,
                            int64_t nrows, int nsb, uint8_t *dst, hipStream_t st) {
  int64_t n = nrows * nsb;
  int threads = 128;
  int64_t blocks = (n + threads - 1) / threads;
  hipLaunchKernelGGL(k_repack, dim3((unsigned)blocks), dim3(threads), 0, st, type, srcs_dev,
                     rowmap, nrows, nsb, dst);
  return hipGetLastError();
}
