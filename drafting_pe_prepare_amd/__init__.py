"""MI355X-native P-EAGLE parallel-draft step.

The compute lives in libpe.so (HIP for gfx950, C ABI in include/pe.h);
`drafting_pe_prepare_amd.binding` marshals arguments to it.  Importing this
package loads nothing: `configs` and `synth` (workload shapes and seeded
inputs) work without a GPU.
"""
