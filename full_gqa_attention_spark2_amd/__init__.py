"""MI355X-native hybrid sliding/full GQA attention core.

The compute path is the HIP library ``libhattn.so`` built from ``csrc/``;
``binding`` marshals torch tensors into its C-ABI. Importing this package
does not load the library; ``binding.lib()`` does, and fails loudly when the
library is missing.
"""
