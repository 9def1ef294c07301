// Row copies between a sequence's last, shorter chunk and a zero-padded
// one-chunk buffer.  A sequence whose length is not a multiple of the chunk
// length Q runs its whole chunks in place and its remaining tokens as one
// chunk of Q rows, the rows past the sequence's end set to zero: a zero step
// size leaves the state and the chunk's cumulative decay unchanged, and zero
// x, B, C and dy rows contribute nothing to any output or gradient.
//
// Rows are `rowbytes` bytes; sequence b's rows start at row b * L of the
// strided tensor and at row b * Q of the padded buffer.  The copies work in
// the widest unit (16, 8, 4 or 2 bytes) that divides the row size; both base
// pointers are 16-byte aligned.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.h"

namespace ssd {
namespace {

template <typename U>
__global__ __launch_bounds__(256) void k_pad_rows(const U* __restrict__ src, U* __restrict__ dst, int64_t rowlen,
                                                  int64_t L, int64_t row0, int64_t nvalid, int64_t Q,
                                                  int64_t total) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = e / rowlen, col = e - r * rowlen;
    const int64_t b = r / Q, i = r - b * Q;
    U v{};
    if (i < nvalid) v = src[(b * L + row0 + i) * rowlen + col];
    dst[e] = v;
  }
}

template <typename U>
__global__ __launch_bounds__(256) void k_unpad_rows(const U* __restrict__ src, U* __restrict__ dst, int64_t rowlen,
                                                    int64_t L, int64_t row0, int64_t nvalid, int64_t Q,
                                                    int64_t total) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = e / rowlen, col = e - r * rowlen;
    const int64_t b = r / nvalid, i = r - b * nvalid;
    dst[(b * L + row0 + i) * rowlen + col] = src[(b * Q + i) * rowlen + col];
  }
}

template <typename U>
void launch(bool pad, const void* src, void* dst, int64_t rowbytes, int64_t L, int64_t row0, int64_t nvalid,
            int64_t Q, int64_t b, hipStream_t st) {
  const int64_t rowlen = rowbytes / (int64_t)sizeof(U);
  const int64_t total = b * (pad ? Q : nvalid) * rowlen;
  if (total <= 0) return;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (pad)
    k_pad_rows<U><<<dim3((unsigned)blocks), dim3(256), 0, st>>>(static_cast<const U*>(src), static_cast<U*>(dst),
                                                                rowlen, L, row0, nvalid, Q, total);
  else
    k_unpad_rows<U><<<dim3((unsigned)blocks), dim3(256), 0, st>>>(static_cast<const U*>(src), static_cast<U*>(dst),
                                                                  rowlen, L, row0, nvalid, Q, total);
}

void dispatch(bool pad, const void* src, void* dst, int64_t rowbytes, int64_t L, int64_t row0, int64_t nvalid,
              int64_t Q, int64_t b, hipStream_t st) {
  if (rowbytes % 16 == 0) launch<uint4>(pad, src, dst, rowbytes, L, row0, nvalid, Q, b, st);
  else if (rowbytes % 8 == 0) launch<uint2>(pad, src, dst, rowbytes, L, row0, nvalid, Q, b, st);
  else if (rowbytes % 4 == 0) launch<uint32_t>(pad, src, dst, rowbytes, L, row0, nvalid, Q, b, st);
  else launch<uint16_t>(pad, src, dst, rowbytes, L, row0, nvalid, Q, b, st);
}

}  // namespace

void pad_rows(const void* src, void* dst, int64_t rowbytes, int64_t L, int64_t row0, int64_t nvalid, int64_t Q,
              int64_t b, hipStream_t st) {
  dispatch(true, src, dst, rowbytes, L, row0, nvalid, Q, b, st);
}

void unpad_rows(const void* src, void* dst, int64_t rowbytes, int64_t L, int64_t row0, int64_t nvalid, int64_t Q,
                int64_t b, hipStream_t st) {
  dispatch(false, src, dst, rowbytes, L, row0, nvalid, Q, b, st);
}

}  // namespace ssd
