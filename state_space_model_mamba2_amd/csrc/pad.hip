// Row copies between a sequence's last, shorter chunk and a zero-padded
// one-chunk buffer.  A sequence whose length is not a multiple of the chunk
// length Q has its last chunk read from and written to such buffers of Q
// rows, the rows past the sequence's end set to zero: a zero step size
// leaves the state and the chunk's cumulative decay unchanged, and zero x, B,
// C and dy rows contribute nothing to any output or gradient.
//
// Sequence b's rows start at row b * L of the strided tensor and at row b * Q
// of the padded buffer.  One launch copies up to four tensors (blockIdx.y
// picks the tensor), each in the widest unit (16, 8, 4 or 2 bytes) that
// divides its row size; every pointer is 16-byte aligned.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.h"

namespace ssd {
namespace {

struct CopyJob {
  const char* src[4];
  char* dst[4];
  int64_t rowbytes[4];
  int64_t L, row0, nvalid, Q;
};

template <typename U, bool PAD>
__device__ void copy_rows(const CopyJob& j, int t, int64_t nb) {
  const int64_t rowlen = j.rowbytes[t] / (int64_t)sizeof(U);
  const U* src = reinterpret_cast<const U*>(j.src[t]);
  U* dst = reinterpret_cast<U*>(j.dst[t]);
  const int64_t rows = PAD ? j.Q : j.nvalid;  // per sequence
  const int64_t total = nb * rows * rowlen;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = e / rowlen, col = e - r * rowlen;
    const int64_t b = r / rows, i = r - b * rows;
    const int64_t strided = (b * j.L + j.row0 + i) * rowlen + col;
    const int64_t padded = (b * j.Q + i) * rowlen + col;
    if (PAD) {
      U v{};
      if (i < j.nvalid) v = src[strided];
      dst[padded] = v;
    } else {
      dst[strided] = src[padded];
    }
  }
}

template <bool PAD>
__global__ __launch_bounds__(256) void k_copy_rows(const CopyJob j, int64_t nb) {
  const int t = blockIdx.y;
  const int64_t rb = j.rowbytes[t];
  if (rb % 16 == 0) copy_rows<uint4, PAD>(j, t, nb);
  else if (rb % 8 == 0) copy_rows<uint2, PAD>(j, t, nb);
  else if (rb % 4 == 0) copy_rows<uint32_t, PAD>(j, t, nb);
  else copy_rows<uint16_t, PAD>(j, t, nb);
}

template <bool PAD>
void launch(const RowCopy& c, int64_t L, int64_t row0, int64_t nvalid, int64_t Q, int64_t b, hipStream_t st) {
  if (c.n <= 0) return;
  CopyJob j{};
  int64_t most = 0;
  for (int t = 0; t < c.n; ++t) {
    j.src[t] = static_cast<const char*>(c.src[t]);
    j.dst[t] = static_cast<char*>(c.dst[t]);
    j.rowbytes[t] = c.rowbytes[t];
    const int64_t units = b * (PAD ? Q : nvalid) * c.rowbytes[t] / 16;
    if (units > most) most = units;
  }
  j.L = L; j.row0 = row0; j.nvalid = nvalid; j.Q = Q;
  int64_t blocks = (most + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 2048) blocks = 2048;
  k_copy_rows<PAD><<<dim3((unsigned)blocks, (unsigned)c.n), dim3(256), 0, st>>>(j, b);
}

}  // namespace

void pad_rows(const RowCopy& c, int64_t L, int64_t row0, int64_t nvalid, int64_t Q, int64_t b, hipStream_t st) {
  launch<true>(c, L, row0, nvalid, Q, b, st);
}

void unpad_rows(const RowCopy& c, int64_t L, int64_t row0, int64_t nvalid, int64_t Q, int64_t b, hipStream_t st) {
  launch<false>(c, L, row0, nvalid, Q, b, st);
}

}  // namespace ssd
