// Arguments of the LDS-tiled matrix-core kernel (internal).
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace brq {

enum { EPI_Y = 0, EPI_HS32 = 1, EPI_PAIRSUM = 2 };

struct TileArgs {
  const void* a;            // activations: permuted fp16 [M][K]
  int M, N, K;              // A rows, output columns, reduction length
  const uint64_t* signs;    // SIGN1 plane [N][K/64]
  const uint16_t* scales;   // group-128 scales [N][K/128] (BM_GROUP)
  const uint16_t* kmag;     // fp16 per-k magnitudes [K], natural order (BM_PERK)
  const uint16_t* diag;     // fp16 per-column diagonal (EPI_HS32, EPI_PAIRSUM)
  const int* rexp;          // EPI_PAIRSUM: per-token exponent applied to the piece sum (2^rexp);
                            // EPI_HS32: per-row staging exponent undone (2^-rexp)
  void* out;
  int out_bf16;
  int ksplit = 1;           // K-slices (grid y); EPI_HS32 writes slice s at out + s*M*N
};

int dbf1_ksplit(int M, int r, int n);

hipError_t launch_tile_dbf1(const TileArgs& a, hipStream_t st);
hipError_t launch_tile_dbf2(const TileArgs& a, hipStream_t st);

}  // namespace brq
