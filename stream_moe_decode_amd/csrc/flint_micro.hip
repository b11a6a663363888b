// Measurement helpers reported beside the decode numbers (not part of the decode path): a streaming
// read (the practical HBM ceiling), rounds of a tagged all-to-all exchange among co-resident workgroups
// (the cost of one of the decode kernel's cross-workgroup hand-offs), and back-to-back empty launches
// (the cost a kernel boundary adds), the three microbenchmarks that "Flint Inference on Apple Silicon:
// rec Megakernel and Tempo9 Compared" sets beside its decode measurements (section 3).
#include "flint_internal.h"
#include "flint_device.h"

namespace flint {
namespace {

// Every byte of p once, the way the decode kernel brings its weights in: workgroup g streams its
// contiguous share with direct-to-LDS loads of 1 KB per wave instruction, 8 to 16 of them in flight per
// wave (a rolling window over a 16 KB LDS ring per wave whose contents are never used; one word of it is
// stored only if it equals a value zeroed memory cannot give).
__global__ void __launch_bounds__(256) micro_read(const uint8_t* p, size_t per, uint32_t* sink) {
  __shared__ uint4 ring[4][16 * 64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint8_t* base = p + (size_t)blockIdx.x * per;
  const size_t units = per / 1024;
  int k = 0;
  for (size_t u = wave; u < units; u += 4, ++k) {
    dma16(base + u * 1024 + lane * 16, &ring[wave][(k & 15) * 64]);
    if ((k & 7) == 7) wait_vmem_n<8>();
  }
  wait_vmem();
  __syncthreads();
  if (ring[0][threadIdx.x].x == 0x9E3779B9u) gp(sink)[0] = 1u;
}

// `rounds` all-to-all exchanges in the decode kernel's form: workgroup w publishes (round << 32 | w) in
// slot w of each of the NCOPY replicas (one per XCD; lane c stores replica c) with system-scope stores,
// then thread t reads slot t of replica w % NCOPY (every slot at once) and re-polls it until it carries
// at least that round.  Each wait is bounded: past the bound the kernel latches *err and the workgroup
// leaves, so every workgroup finishes.
__global__ void __launch_bounds__(256) micro_exchange(unsigned long long* slots, int rounds, uint32_t* err) {
  __shared__ int bad;
  const int W = blockIdx.x, G = gridDim.x, tid = threadIdx.x;
  const unsigned long long* mine = slots + (size_t)(W % NCOPY) * G;
  if (tid == 0) bad = 0;
  __syncthreads();
  for (int r = 1; r <= rounds; ++r) {
    if (tid < NCOPY)
      __hip_atomic_store(gp(slots) + (size_t)tid * G + W, ((unsigned long long)r << 32) | (unsigned)W,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    for (int s = tid; s < G; s += 256) {
      int polls = 0;
      while ((int)(__hip_atomic_load(gp(mine) + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) >> 32) < r)
        if (++polls > (1 << 20)) {
          __hip_atomic_fetch_or(gp(err), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
          bad = 1;
          break;
        }
    }
    __syncthreads();
    if (bad) return;
  }
}

// The same round confined to each XCD: workgroup W belongs to group W % 8 (the XCD the dispatcher places
// it on), writes one slot of its group with a device-scope store (it stays in the XCD's L2) and polls the
// G / 8 slots of its group with device-scope loads.
__global__ void __launch_bounds__(256) micro_exchange_xcd(unsigned long long* slots, int rounds, uint32_t* err) {
  __shared__ int bad;
  const int W = blockIdx.x, G = gridDim.x, tid = threadIdx.x;
  unsigned long long* const grp = slots + (size_t)(W % NCOPY) * G;
  if (tid == 0) bad = 0;
  __syncthreads();
  for (int r = 1; r <= rounds; ++r) {
    if (tid == 0)
      __hip_atomic_store(gp(grp) + W, ((unsigned long long)r << 32) | (unsigned)W, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    for (int s = W % NCOPY + NCOPY * tid; s < G; s += NCOPY * 256) {
      int polls = 0;
      while ((int)(__hip_atomic_load(gp(grp) + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >> 32) < r)
        if (++polls > (1 << 20)) {
          __hip_atomic_fetch_or(gp(err), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
          bad = 1;
          break;
        }
    }
    __syncthreads();
    if (bad) return;
  }
}

__global__ void micro_empty() {}

}  // namespace

hipError_t launch_micro_read(const void* p, size_t bytes, uint32_t* sink, int blocks, hipStream_t st) {
  const size_t per = bytes / blocks / 1024 * 1024;  // whole 1 KB units per workgroup
  hipLaunchKernelGGL(micro_read, dim3(blocks), dim3(256), 0, st, (const uint8_t*)p, per, sink);
  return hipGetLastError();
}
hipError_t launch_micro_exchange(unsigned long long* slots, int workgroups, int rounds, uint32_t* err, hipStream_t st,
                                 bool xcd) {
  if (xcd)
    hipLaunchKernelGGL(micro_exchange_xcd, dim3(workgroups), dim3(256), 0, st, slots, rounds, err);
  else
    hipLaunchKernelGGL(micro_exchange, dim3(workgroups), dim3(256), 0, st, slots, rounds, err);
  return hipGetLastError();
}
hipError_t launch_micro_empty(hipStream_t st) {
  hipLaunchKernelGGL(micro_empty, dim3(1), dim3(64), 0, st);
  return hipGetLastError();
}

}  // namespace flint
