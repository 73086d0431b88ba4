// Calibration probes for the benchmark (not part of the TQ2_0 ABI): an empty
// kernel (dispatch floor), read-only streaming kernels (the achievable HBM
// read rate at a given byte count, dispatch included) and a write-only fill
// (used to scale hardware write counters).  Built into libtq2probe.so.
//
// Read kernels (all fold what they read into one value that is stored only
// if it equals a value no input produces, so no load can be removed):
//   grid-stride : a fixed grid; each thread walks the buffer with stride
//                 grid*256 words, U loads in flight per pass, non-temporal;
//   blocked     : the grid is sized from the byte count so that every thread
//                 issues exactly U 16-byte loads, all before it consumes
//                 any; workgroup b reads one contiguous run of 256*U words
//                 and every wave instruction reads 1 KiB contiguous (the
//                 matvec's own pattern).  Variants: raw buffer loads
//                 (scalar descriptor, 32-bit lane offsets, reads past the
//                 end return 0) or global loads; non-temporal or default
//                 cache policy; or straight to LDS (buffer_load ... lds).
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

__global__ void k_empty() {}

__device__ __forceinline__ uint32_t fold(v4u a) { return a.x ^ a.y ^ a.z ^ a.w; }

__global__ __launch_bounds__(256) void k_read(const v4u* __restrict__ p, int64_t n16,
                                              uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const v4u a = __builtin_nontemporal_load(p + i);
    const v4u b = __builtin_nontemporal_load(p + i + stride);
    const v4u c = __builtin_nontemporal_load(p + i + 2 * stride);
    const v4u d = __builtin_nontemporal_load(p + i + 3 * stride);
    acc ^= fold(a) ^ fold(b) ^ fold(c) ^ fold(d);
  }
  for (; i < n16; i += stride) acc ^= fold(__builtin_nontemporal_load(p + i));
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// blocked read, MODE 0: raw buffer loads, 1: global loads; NT: non-temporal
// policy.  Thread t of workgroup b reads words b*256*U + 256*j + t.
template <int U, int MODE, bool NT>
__global__ __launch_bounds__(256) void k_read_blk(const v4u* __restrict__ p, int64_t n16,
                                                  uint32_t* __restrict__ sink) {
  const int64_t base = (int64_t)blockIdx.x * 256 * U + threadIdx.x;
  v4u v[U];
  if constexpr (MODE == 0) {
    // descriptor over this workgroup's run (at most 256*U words, clipped)
    const int64_t w0 = (int64_t)blockIdx.x * 256 * U;
    const int64_t left = n16 - w0;
    const uint32_t bytes = (uint32_t)((left < 256 * U ? left : 256 * U) * 16);
    const __amdgpu_buffer_rsrc_t r = rsrc(p + w0, bytes);
#pragma unroll
    for (int j = 0; j < U; ++j)
      v[j] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(
                                         r, (int)((256 * j + threadIdx.x) * 16), 0, NT ? 2 : 0));
  } else {
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t i = base + 256 * j;
      const int64_t ic = i < n16 ? i : n16 - 1;  // in bounds, unconditional
      v[j] = NT ? __builtin_nontemporal_load(p + ic) : p[ic];
    }
  }
  uint32_t acc = 0;
#pragma unroll
  for (int j = 0; j < U; ++j) acc ^= fold(v[j]);
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

// blocked read straight to LDS: each wave's U loads of 1 KiB land in its own
// LDS region; after they complete one dword per load is read back.
template <int U>
__global__ __launch_bounds__(256) void k_read_blk_lds(const v4u* __restrict__ p, int64_t n16,
                                                      uint32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[4 * U * 1024];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t w0 = (int64_t)blockIdx.x * 256 * U;
  const int64_t left = n16 - w0;
  const uint32_t bytes = (uint32_t)((left < 256 * U ? left : 256 * U) * 16);
  const __amdgpu_buffer_rsrc_t r = rsrc(p + w0, bytes);
  uint8_t* mine = lds + wave * U * 1024;
#pragma unroll
  for (int j = 0; j < U; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(mine + 1024 * j), 16,
                                             (int)((256 * j + threadIdx.x) * 16), 0, 0, 2);
  __builtin_amdgcn_s_waitcnt(0);  // every counter drained: the LDS writes have landed
  __builtin_amdgcn_wave_barrier();
  uint32_t acc = 0;
#pragma unroll
  for (int j = 0; j < U; ++j) acc ^= reinterpret_cast<const uint32_t*>(mine + 1024 * j)[lane];
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

__global__ __launch_bounds__(256) void k_fill(uint4* __restrict__ p, int64_t n16, uint32_t v) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(v, v, v, v);
}

template <int U>
hipError_t launch_blk(int mode, int nt, const v4u* p, int64_t n16, uint32_t* sink, hipStream_t s) {
  const int64_t per = 256LL * U;
  const dim3 grid((unsigned)((n16 + per - 1) / per));
  if (mode == 2) {
    hipLaunchKernelGGL((k_read_blk_lds<U>), grid, dim3(256), 0, s, p, n16, sink);
  } else if (mode == 0) {
    if (nt) hipLaunchKernelGGL((k_read_blk<U, 0, true>), grid, dim3(256), 0, s, p, n16, sink);
    else hipLaunchKernelGGL((k_read_blk<U, 0, false>), grid, dim3(256), 0, s, p, n16, sink);
  } else {
    if (nt) hipLaunchKernelGGL((k_read_blk<U, 1, true>), grid, dim3(256), 0, s, p, n16, sink);
    else hipLaunchKernelGGL((k_read_blk<U, 1, false>), grid, dim3(256), 0, s, p, n16, sink);
  }
  return hipGetLastError();
}

}  // namespace

extern "C" {

int32_t tq2probe_empty(void* stream) {
  hipLaunchKernelGGL(k_empty, dim3(1), dim3(64), 0, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

// The empty kernel with `id` (1..65535) workgroups of 64 threads: a marker
// whose grid size names a section of a kernel trace.
int32_t tq2probe_marker(int32_t id, void* stream) {
  if (id < 1 || id > 65535) return 1;
  hipLaunchKernelGGL(k_empty, dim3((unsigned)id), dim3(64), 0, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

// Grid-stride read: `blocks` workgroups of 256 threads, 4 non-temporal loads
// in flight per pass while four strides remain, then one per pass.  bytes
// must be a multiple of 16 and p 16-byte aligned; sink holds `blocks`
// uint32 (written only in the impossible case).
int32_t tq2probe_read_gridstride(const void* p, int64_t bytes, uint32_t* sink, int32_t blocks, void* stream) {
  if (!p || !sink || bytes <= 0 || bytes % 16 || ((uintptr_t)p % 16) || blocks < 1) return 1;
  hipLaunchKernelGGL(k_read, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const v4u*)p, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

// Number of workgroups tq2probe_read_blocked launches for these arguments
// (the size of `sink` it needs, in uint32), or 0 for invalid ones.
int64_t tq2probe_blocked_grid(int64_t bytes, int32_t loads) {
  if (bytes <= 0 || bytes % 16 || (loads != 1 && loads != 2 && loads != 4 && loads != 8 && loads != 16))
    return 0;
  const int64_t per = 256LL * loads;
  return (bytes / 16 + per - 1) / per;
}

// Blocked read (see above): `loads` (1, 2, 4, 8, 16) 16-byte loads per
// thread, all in flight at once; mode 0 = raw buffer loads, 1 = global
// loads, 2 = straight to LDS (buffer loads, non-temporal); nt = non-temporal
// cache policy (modes 0 and 1).  The buffer must be at most 2^31 - 1 bytes
// per workgroup run (always true) and p 16-byte aligned; sink holds
// tq2probe_blocked_grid(bytes, loads) uint32.
int32_t tq2probe_read_blocked(const void* p, int64_t bytes, uint32_t* sink, int32_t loads, int32_t mode,
                              int32_t nt, void* stream) {
  if (!p || !sink || ((uintptr_t)p % 16) || mode < 0 || mode > 2 || tq2probe_blocked_grid(bytes, loads) == 0)
    return 1;
  const v4u* q = (const v4u*)p;
  const int64_t n16 = bytes / 16;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  switch (loads) {
    case 1: e = launch_blk<1>(mode, nt, q, n16, sink, s); break;
    case 2: e = launch_blk<2>(mode, nt, q, n16, sink, s); break;
    case 4: e = launch_blk<4>(mode, nt, q, n16, sink, s); break;
    case 8: e = launch_blk<8>(mode, nt, q, n16, sink, s); break;
    default: e = launch_blk<16>(mode, nt, q, n16, sink, s); break;
  }
  return e == hipSuccess ? 0 : 6;
}

// The read-only stream the benchmark sets beside every matvec: the fastest
// variant of the sweep at the matvec sizes on MI355X (blocked, one 16-byte
// non-temporal global load per thread, grid sized from the byte count).
// sink holds tq2probe_blocked_grid(bytes, 1) uint32.
int32_t tq2probe_read(const void* p, int64_t bytes, uint32_t* sink, void* stream) {
  return tq2probe_read_blocked(p, bytes, sink, 1, 1, 1, stream);
}

int32_t tq2probe_fill(void* p, int64_t bytes, uint32_t value, int32_t blocks, void* stream) {
  if (!p || bytes <= 0 || bytes % 16 || ((uintptr_t)p % 16) || blocks < 1) return 1;
  hipLaunchKernelGGL(k_fill, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (uint4*)p,
                     bytes / 16, value);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

}  // extern "C"
