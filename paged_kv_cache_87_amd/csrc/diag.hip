// Read-bandwidth probe.  The decode reads each K/V byte once, so its practical
// ceiling on this device is the rate of a plain read stream, not the HBM
// peak; this kernel is that stream.  Each workgroup XORs the 32-bit words of
// one contiguous share of a buffer with non-temporal 16-byte loads (the
// decode's load kind), reduces them across its waves and writes one word, so
// the result is a checksum the host can verify.

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kDiagThreads = 256;
constexpr int kDiagUnroll = 4;

__global__ __launch_bounds__(kDiagThreads) void read_checksum_kernel(ReadChecksumArgs a) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  __shared__ uint32_t sm[kDiagThreads / 64];
  const uint64_t lo = a.chunks_per_word * blockIdx.x;
  const uint64_t hi = lo + a.chunks_per_word < a.chunks ? lo + a.chunks_per_word : a.chunks;
  const uint32_t n = lo < hi ? static_cast<uint32_t>(hi - lo) : 0u;
  // the share's bytes; loads past them return zeros (size checked on the host)
  const Rsrc r = make_rsrc(static_cast<const char*>(a.buf) + lo * 16, n * 16u);
  uint32_t acc = 0;
  for (uint32_t i = threadIdx.x; i < n; i += kDiagThreads * kDiagUnroll) {
    u32x4 v[kDiagUnroll];
#pragma unroll
    for (int u = 0; u < kDiagUnroll; ++u)
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, (i + kDiagThreads * u) * 16u, 0, 2);
#pragma unroll
    for (int u = 0; u < kDiagUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(acc), m));
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) a.words[blockIdx.x] = sm[0] ^ sm[1] ^ sm[2] ^ sm[3];
}

}  // namespace

hipError_t launch_read_checksum(const ReadChecksumArgs& a, int num_words, hipStream_t stream) {
  return launch_kernel(read_checksum_kernel, dim3(num_words), dim3(kDiagThreads), 0, stream, a);
}

}  // namespace pa
